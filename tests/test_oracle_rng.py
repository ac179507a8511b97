"""Pins of the oracle's random-number and logarithm code (CPU only).

Philox4x32-10 follows Salmon et al., "Parallel Random Numbers: As Easy as 1,
2, 3" (SC'11).  Its round structure is pinned by running the same generic
definition at word width 64 against numpy's Philox4x64-10 bit generator; the
bulk numpy version is pinned against the generic one.  The fp32 logarithm is
pinned by brute force over every input the sampler can produce."""
import numpy as np
import pytest
from scipy import stats

from oracle import rng
from oracle.sampler import gumbel_argmax


def test_philox_round_structure_matches_numpy_philox4x64():
    # numpy's Philox advances its 256-bit counter before producing a block, so
    # the block produced from state counter c is Philox(c + 1).
    for ctr, key in [([0, 0, 0, 0], [0, 0]), ([5, 7, 9, 11], [123, 456]),
                     ([2**64 - 1, 3, 1, 2**63], [2**64 - 1, 17])]:
        bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64),
                              key=np.array(key, dtype=np.uint64))
        got = [int(x) for x in bg.random_raw(4)]
        c = list(ctr)
        c[0] = (c[0] + 1) % 2**64
        if c[0] == 0:
            c[1] += 1
        assert got == rng.philox_generic(c, key, rng.PHILOX4x64)


def test_philox4x32_vectorised_equals_definition():
    g = np.random.default_rng(0)
    c = g.integers(0, 2**32, size=(4, 64), dtype=np.uint64)
    k = g.integers(0, 2**32, size=(2, 64), dtype=np.uint64)
    v = rng.philox4x32(c[0], c[1], c[2], c[3], k[0], k[1])
    for i in range(64):
        assert [int(v[j][i]) for j in range(4)] == rng.philox_generic(c[:, i], k[:, i])


def test_philox_rounds_matter():
    # fewer rounds give different words: the loop really runs 10 rounds
    a = rng.philox_generic([1, 2, 3, 4], [5, 6])
    b = rng.philox_generic([1, 2, 3, 4], [5, 6], rounds=9)
    assert a != b


def test_philox4x32_words_uniform():
    n = 1 << 16
    ctr = np.arange(n, dtype=np.uint64)
    words = np.concatenate(rng.philox4x32(ctr, 3, 7, 0, 0x1234, 0x5678))
    counts = np.bincount((words >> np.uint32(24)).astype(np.int64), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4
    bits = np.unpackbits(words.view(np.uint8))
    assert abs(bits.mean() - 0.5) < 3e-3


def test_uniform_open01_exact_endpoints_and_symmetry():
    x = np.array([0, 0xFFFFFFFF, 0x1FF, 0x200, 0x80000000], dtype=np.uint32)
    u = rng.uniform_open01(x)
    assert u[0] == np.float32(2.0 ** -24)
    assert u[1] == np.float32(1.0 - 2.0 ** -24)
    assert u[2] == u[0] and u[3] == np.float32(3 * 2.0 ** -24)
    assert u[4] == np.float32(0.5 + 2.0 ** -24)
    w = np.random.default_rng(1).integers(0, 2**32, size=10000, dtype=np.uint64).astype(np.uint32)
    assert np.all(rng.uniform_open01(w) + rng.uniform_open01(~w) == np.float32(1.0))
    assert np.all((rng.uniform_open01(w) > 0) & (rng.uniform_open01(w) < 1))


def _ulp_err(got, ref):
    got = np.asarray(got, np.float32)
    return np.abs(got.astype(np.float64) - ref) / np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)


def test_ln_f32_brute_force_all_sampler_inputs():
    # every u the sampler can draw: (2k + 1) 2^-24, k = 0 .. 2^23 - 1
    u = ((np.arange(1 << 23, dtype=np.uint32) * np.uint32(2) + np.uint32(1)).astype(np.float32)
         * np.float32(2.0 ** -24))
    a = rng.ln_f32(u)
    err1 = _ulp_err(a, np.log(u.astype(np.float64)))
    b = -a
    c = rng.ln_f32(b)
    err2 = _ulp_err(c, np.log(b.astype(np.float64)))
    assert err1.max() <= 3.0, err1.max()
    assert err2.max() <= 3.0, err2.max()


def test_ln_f32_wide_range_and_special_values():
    g = np.random.default_rng(2)
    x = np.exp(g.uniform(-80, 80, size=200000)).astype(np.float32)
    err = _ulp_err(rng.ln_f32(x), np.log(x.astype(np.float64)))
    assert err.max() <= 3.0
    assert rng.ln_f32(np.float32([1.0]))[0] == 0.0
    assert rng.ln_f32(np.float32([2.0]))[0] == np.float32(np.log(2.0))
    # monotone on a fine grid around 1
    x = np.float32(1.0) + np.arange(-2000, 2000, dtype=np.float32) * np.float32(2.0 ** -20)
    assert np.all(np.diff(rng.ln_f32(x)) >= 0)


def test_gumbel_max_frequencies_match_softmax():
    V, tau = 8, 0.7
    l = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4, 0.9, 1.5], dtype=np.float32)
    inv = np.float32(1.0 / tau)
    groups, steps = 1024, 128
    v = np.arange(V, dtype=np.uint64)[:, None, None]
    g = np.arange(groups, dtype=np.uint64)[None, :, None]
    s = np.arange(steps, dtype=np.uint64)[None, None, :]
    words = rng.philox4x32(v, g, s, 0, 0xDEADBEEF, 0x01234567)
    a = (l * inv).astype(np.float32)[:, None, None]
    counts = np.zeros(V, np.int64)
    for w in words:
        score = a + rng.gumbel_f32(rng.uniform_open01(w))
        counts += np.bincount(np.argmax(score, axis=0).ravel(), minlength=V)
    p = np.exp(l.astype(np.float64) * float(inv))
    p /= p.sum()
    assert counts.sum() == 4 * groups * steps
    assert stats.chisquare(counts, p * counts.sum()).pvalue > 1e-4


def test_gumbel_argmax_small_temperature_is_argmax():
    g = np.random.default_rng(3)
    l = g.standard_normal((12, 300)).astype(np.float32) * 4
    xhat, _, _ = gumbel_argmax(l, np.float32(1e4), 99, 5)
    assert np.array_equal(xhat, np.argmax(l, axis=1))


def test_gumbel_argmax_uses_declared_counters():
    # element (i, v) at step s uses counter (v, i >> 2, s, 0), word i & 3
    l = np.zeros((6, 16), np.float32)
    seed = (7 << 32) | 11
    xhat, best, _ = gumbel_argmax(l, np.float32(1.0), seed, 3)
    for i in range(6):
        ws = [rng.philox_generic([v, i >> 2, 3, 0], [11, 7])[i & 3] for v in range(16)]
        gs = rng.gumbel_f32(rng.uniform_open01(np.array(ws, np.uint32)))
        assert xhat[i] == int(np.argmax(gs)) and best[i] == gs.max()


def test_uniform_index_power_of_two_is_top_bits():
    w = np.random.default_rng(4).integers(0, 2**32, size=5000, dtype=np.uint64)
    for V in (2048, 262144):
        assert np.array_equal(rng.uniform_index(w, V), (w >> (32 - int(np.log2(V)))).astype(np.int64))
    counts = np.bincount(rng.uniform_index(
        np.concatenate(rng.philox4x32(np.arange(40000, dtype=np.uint64), 0, 0, 1, 5, 6)), 50),
        minlength=50)
    assert stats.chisquare(counts).pvalue > 1e-4


def test_weyl_constants_from_closed_forms():
    # The key schedule adds the golden ratio's fractional part and sqrt(3) - 1,
    # scaled to the word width and truncated (SC'11, section 3, Philox key
    # schedule).  Derived here in exact integer arithmetic.
    from math import isqrt
    for params in (rng.PHILOX4x32, rng.PHILOX4x64):
        w = params["w"]
        # floor(2^w (sqrt(5) - 1) / 2): sqrt(5) * 2^w = isqrt(5 * 4^w) (floor)
        phi = (isqrt(5 << (2 * w)) - (1 << w)) >> 1
        # floor(2^w (sqrt(3) - 1))
        s3 = isqrt(3 << (2 * w)) - (1 << w)
        assert params["k"] == (phi, s3), (w, hex(phi), hex(s3))


def _rocrand_kat_binary(tmp_path_factory):
    """A host program built from ROCm's rocRAND Philox4x32-10 header: an
    independent implementation of the generator (source shipped with ROCm)."""
    import os
    import shutil
    import subprocess
    inc = "/opt/rocm/include"
    hdr = os.path.join(inc, "rocrand", "rocrand_philox4x32_10.h")
    gxx = shutil.which("g++")
    if not os.path.exists(hdr) or gxx is None:
        pytest.skip("rocRAND header or g++ not available")
    d = tmp_path_factory.mktemp("rocrand_kat")
    src = d / "kat.cpp"
    src.write_text(
        "#include <rocrand/rocrand_philox4x32_10.h>\n"
        "#include <cstdio>\n#include <cstdlib>\n"
        "int main(int argc, char** argv) {\n"
        "  for (int a = 1; a + 2 < argc; a += 3) {\n"
        "    rocrand_device::philox4x32_10_engine e(strtoull(argv[a], 0, 0), strtoull(argv[a + 1], 0, 0),\n"
        "                                            strtoull(argv[a + 2], 0, 0));\n"
        "    for (int i = 0; i < 4; ++i) printf(\"%u \", e());\n"
        "    printf(\"\\n\");\n"
        "  }\n"
        "}\n")
    exe = d / "kat"
    r = subprocess.run([gxx, "-O1", "-D__HIP_PLATFORM_AMD__", "-I", inc, str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("rocRAND header does not build on the host: " + r.stderr[-300:])
    return exe


def test_philox4x32_matches_rocrand(tmp_path_factory):
    # rocRAND's engine seeded with (seed, subsequence, offset) produces, as its
    # first four words, Philox4x32-10 of counter (offset / 4 as two words,
    # subsequence as two words) under key (seed low word, seed high word).
    # This pins the 4x32 multipliers, which numpy's 4x64 generator does not.
    import subprocess
    exe = _rocrand_kat_binary(tmp_path_factory)
    g = np.random.default_rng(5)
    cases = [(0, 0, 0), (0x123456789, 5, 8), (2**64 - 1, 2**64 - 1, 4 * (2**64 // 4 - 1))]
    for _ in range(40):
        cases.append((int(g.integers(0, 2**63)) * 2 + 1, int(g.integers(0, 2**63)),
                      4 * int(g.integers(0, 2**61))))
    args = [str(x) for c in cases for x in c]
    out = subprocess.run([str(exe)] + args, capture_output=True, text=True, check=True).stdout.split("\n")
    for (seed, sub, off), line in zip(cases, out):
        got = [int(x) for x in line.split()]
        c = off // 4
        ctr = [c & 0xFFFFFFFF, c >> 32, sub & 0xFFFFFFFF, sub >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        assert got == rng.philox_generic(ctr, key), (seed, sub, off)
        v = rng.philox4x32(*ctr, *key)
        assert got == [int(x) for x in v]
