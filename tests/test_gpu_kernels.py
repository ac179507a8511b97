"""GPU parity of libdg's building blocks against the CPU oracle (through the C ABI).

* the MFMA GEMM against float64 products of the same bf16 operands;
* the sampler alone (dg_sample_logits) on seeded synthetic logits: sampled
  tokens, argmax, lock masks, stop decisions bit-exact, entropy to fp32
  rounding, at the tiny vocabulary and at the full 262144-entry vocabulary
  with 1 and 4 canvases;
* the initial canvas (Philox counter at step -1) bit-exact."""
import numpy as np
import pytest
import torch

from discrete_diffusion_decoding_amd import dg, synth
from discrete_diffusion_decoding_amd.configs import SamplerParams, TINY
from oracle import sampler as osmp
from tests.gpu_util import announce, dev, host, rel_l2

pytestmark = pytest.mark.gpu


def _bf16(x):
    return synth.f32_to_bf16_bits(x)


# M <= 4 runs on the weight-streaming GEMV kernel (k slices of up to 16, 32
# and 64 steps of 64 columns take 1, 2 and 4 waves per row set), M < 128 on the
# 64-row tile kernel, 128 <= M < 192 on the 8-wave tile kernel, M >= 192 on
# the 256-row one; the cases cover ragged row chunks, ragged weight tiles and
# single-stage K.
@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (2, 200, 1536), (3, 136, 4096), (4, 72, 2816), (1, 8, 704),
                                   (37, 200, 192), (256, 2816, 2816), (300, 1024, 704),
                                   (64, 8, 256), (192, 72, 64), (260, 200, 192), (513, 136, 320),
                                   (256, 520, 384), (200, 300, 4096), (128, 200, 704), (150, 72, 2816)])
def test_gemm_matches_float64(M, N, K):
    announce(f"gemm M={M} N={N} K={K}")
    g = np.random.default_rng(M * 7 + N)
    A = _bf16(g.standard_normal((M, K)).astype(np.float32))
    W = _bf16((0.05 * g.standard_normal((N, K))).astype(np.float32))
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    dg.dg_gemm_bf16(dev(A.view(np.int16)), dev(W.view(np.int16)), out, M, N, K)
    ref = synth.bf16_bits_to_f32(A).astype(np.float64) @ synth.bf16_bits_to_f32(W).astype(np.float64).T
    got = host(out)
    assert np.all(np.isfinite(got))
    assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max() + 1e-6


# The K-major product (the soft-prediction embedding's E [vocab][d] as stored):
# ragged rows (one and several 256-row items), ragged 256-wide column tiles
# (N a multiple of 8), one and many 64-row K stages, odd and even stage counts.
@pytest.mark.parametrize("M,N,K", [(256, 2816, 704), (37, 200, 64), (300, 264, 192), (513, 520, 4096),
                                   (256, 256, 2048), (64, 8, 320)])
def test_gemm_kmajor_matches_float64(M, N, K):
    announce(f"gemm K-major M={M} N={N} K={K}")
    g = np.random.default_rng(M * 11 + N)
    A = _bf16(g.standard_normal((M, K)).astype(np.float32))
    W = _bf16((0.05 * g.standard_normal((K, N))).astype(np.float32))
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    dg.dg_gemm_bf16_kn(dev(A.view(np.int16)), dev(W.view(np.int16)), out, M, N, K)
    ref = synth.bf16_bits_to_f32(A).astype(np.float64) @ synth.bf16_bits_to_f32(W).astype(np.float64)
    got = host(out)
    assert np.all(np.isfinite(got))
    assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max() + 1e-6


def _canvas(B, T, V):
    st = {
        "tokens": torch.zeros(B, T, dtype=torch.int32, device="cuda"),
        "locked": torch.zeros(B, T, dtype=torch.uint8, device="cuda"),
        "entropy": torch.zeros(B, T, dtype=torch.float32, device="cuda"),
        "xhat": torch.zeros(B, T, dtype=torch.int32, device="cuda"),
        "argmax": torch.zeros(B, T, dtype=torch.int32, device="cuda"),
        "stopped": torch.zeros(B, dtype=torch.int32, device="cuda"),
        "steps": torch.zeros(B, dtype=torch.int32, device="cuda"),
    }
    return st


def _run_sampler_case(B, T, V, scale, peaked, steps, sp, seed=5, logits=None):
    if logits is None:
        logits = synth.logits(seed, f"lg{B}x{T}x{V}", (B, T, V), scale=scale, peaked=peaked)
    seeds = synth.row_seeds(seed, B)
    L = dev(logits)
    st = _canvas(B, T, V)
    canvas = dg.make_canvas(st)
    sampler, keep = dg.make_sampler(sp, seeds)
    ws = torch.empty(dg.dg_sample_workspace_bytes(B, T, V), dtype=torch.uint8, device="cuda")
    tokens = np.zeros((B, T), np.int64)
    amax = np.zeros((B, T), np.int64)
    for s in steps:
        announce(f"sample_logits B={B} T={T} V={V} step={s}")
        dg.dg_sample_logits(L, B, T, V, canvas, s, sampler, ws)
        got = {k: host(v) for k, v in st.items()}
        tok_o, amax_o, stop_o, steps_o, info = osmp.sample_step(
            logits, tokens, amax, s > 0, np.zeros(B, bool), np.zeros(B), s, seeds, sp)
        assert np.array_equal(got["xhat"], info["xhat"])
        assert np.array_equal(got["argmax"], amax_o)
        H = info["entropy"]
        assert np.allclose(got["entropy"], H, rtol=2e-5, atol=2e-5)
        near = np.abs(H - sp.lock_thresh) < 1e-4
        if sp.lock_rule == 0:
            assert np.array_equal(got["locked"].astype(bool)[~near], info["lock"][~near])
        else:
            assert np.array_equal(got["locked"].astype(bool), info["lock"])
        mean_near = np.abs(info["mean_entropy"] - sp.stop_thresh) < 1e-5
        assert np.array_equal(got["stopped"].astype(bool)[~mean_near], stop_o[~mean_near])
        assert np.array_equal(got["steps"], np.full(B, s + 1))
        ok_rows = ~mean_near
        lock_agree = np.all(got["locked"].astype(bool) == info["lock"], axis=1)
        for b in np.nonzero(ok_rows & lock_agree)[0]:
            assert np.array_equal(got["tokens"][b], tok_o[b]), b
        # next step: the oracle continues from its own state (equal to the GPU's
        # wherever asserted above); rows are un-stopped on both sides
        tokens, amax = tok_o, amax_o
        st["stopped"].zero_()
        st["tokens"].copy_(torch.as_tensor(tok_o.astype(np.int32)))


@pytest.mark.parametrize("scale,peaked", [(1.0, 0.0), (4.0, 30.0)])
def test_sampler_tiny_vocab_bit_exact(scale, peaked):
    _run_sampler_case(2, 32, 2048, scale, peaked, [0, 1, 30, 47], SamplerParams())


def test_sampler_pages_variant_rules_bit_exact():
    sp = SamplerParams(lock_rule=1, lock_thresh=0.1, stop_rule=1, stop_thresh=0.005)
    _run_sampler_case(1, 64, 2048, 6.0, 60.0, [0, 1, 2], sp, seed=9)


def test_sampler_maximum_batch_and_canvas_bit_exact():
    """The largest shapes the library accepts: 16 canvases of 1024 positions
    (the finishing kernel then runs 1024 threads per row)."""
    _run_sampler_case(16, 1024, 2048, 2.0, 20.0, [0, 5], SamplerParams(), seed=13)


def test_sampler_full_vocab_one_canvas_bit_exact():
    _run_sampler_case(1, 256, 262144, 1.06, 0.0, [1], SamplerParams())


def test_sampler_full_vocab_four_canvases_bit_exact():
    _run_sampler_case(4, 256, 262144, 1.06, 20.0, [3], SamplerParams(), seed=11)


def test_sampler_near_tie_gumbel_winners_bit_exact():
    """Each row holds three entries whose Gumbel-max scores agree to within a
    few ulps (logits built from the oracle's own noise at this step, all others
    far below; two of them 256 apart, so one GPU thread reads both), so the
    winner is decided by the last bits of the exact scores and, on equality,
    by the lower index."""
    from oracle import rng as orng
    B, T, V, step, seed = 1, 32, 2048, 2, 21
    sp = SamplerParams()
    seeds = synth.row_seeds(seed, B)
    _, inv_tau = osmp.temperature(step, sp.tau_start, sp.tau_end, sp.max_steps)
    k0, k1 = orng.seed_key(int(seeds[0]))
    v = np.arange(V, dtype=np.uint64)
    logits = np.full((B, T, V), -30.0, np.float32)
    for g in range(T // 4):
        words = orng.philox4x32(v, g, step, 0, k0, k1)
        for j in range(4):
            i = 4 * g + j
            noise = orng.gumbel_f32(orng.uniform_open01(words[j]))
            v1, v2 = (7 * i + 3) % V, (13 * i + 1000) % V
            v3 = v1 + 256 if v1 % 1024 < 768 else v1 - 256   # read by the same thread as v1
            for vv, off in ((v1, 0), (v2, (i % 5) - 2), (v3, (i % 3) - 1)):
                lv = np.float32((np.float32(10.0) - noise[vv]) / inv_tau)
                for _ in range(abs(off)):
                    lv = np.nextafter(lv, np.float32(np.inf if off > 0 else -np.inf), dtype=np.float32)
                logits[0, i, vv] = lv
    _run_sampler_case(B, T, V, 0.0, 0.0, [step], sp, seed=seed, logits=logits)


def test_init_canvas_bit_exact():
    announce("init_canvas")
    import ctypes as C
    B, T = 3, 256
    seeds = synth.row_seeds(21, B)
    st = _canvas(B, T, TINY.vocab)
    # dg_init_canvas needs only the vocabulary of a model: use a handle on fake weights
    ptrs = (C.c_void_p * TINY.n_layers)(*([0x1000] * TINY.n_layers))
    w = dg.Weights(0x1000, 0x1000, 0x1000, 0x1000, C.cast(ptrs, C.POINTER(C.c_void_p)))
    h = dg.dg_model_create(TINY, w)
    st["stopped"].fill_(1)
    dg.dg_init_canvas(h, dg.make_canvas(st), B, T, seeds)
    got = host(st["tokens"])
    for b in range(B):
        assert np.array_equal(got[b], osmp.init_canvas(seeds[b], T, TINY.vocab))
    assert host(st["stopped"]).sum() == 0
    dg.dg_model_destroy(h)
