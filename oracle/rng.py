"""Counter-based random numbers and the fp32 logarithm used by the sampler.

Test infrastructure only (see oracle/__init__.py).

* Philox4x32-10: the counter-based generator of Salmon, Moraes, Dror and Shaw,
  "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section 3 (Philox
  S-box: two multiply-hi/lo products per round, Weyl-sequence key schedule,
  10 rounds).  `philox_generic` is the definition written once for any word
  width; `philox4x32` is the same arithmetic vectorised with numpy for bulk use.
* The discrete-diffusion sampler needs a Gumbel variate per (position, vocab
  entry).  G = -ln(-ln u) with u in (0, 1) taken from 23 bits of a Philox word.
  `ln_f32` is this project's own fp32 natural logarithm so that the GPU and
  this oracle take every sampling decision on bit-identical numbers: range
  reduction by the float exponent (Cody-Waite split of ln 2), then
  ln m = 2 atanh(t), t = (m - 1)/(m + 1), m in [sqrt(1/2), sqrt(2)), summed as
  the odd series t + t^3/3 + ... + t^11/11 in Horner form.  Every operation is
  a single IEEE fp32 operation (no fused multiply-add), in a fixed order.
"""
from __future__ import annotations

import numpy as np

U32 = np.uint32
MASK32 = 0xFFFFFFFF

# Philox multipliers and Weyl key increments (SC'11 paper, Philox-4xW).
PHILOX4x32 = dict(w=32, m=(0xD2511F53, 0xCD9E8D57), k=(0x9E3779B9, 0xBB67AE85))
PHILOX4x64 = dict(w=64, m=(0xD2E7470EE14C6C93, 0xCA5A826395121157),
                  k=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B))


def philox_generic(ctr, key, params=PHILOX4x32, rounds: int = 10):
    """Philox-4xW on Python ints: ctr = 4 words, key = 2 words -> 4 words.

    One round: (x0, x1, x2, x3) -> (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2),
    hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)); between rounds the key is bumped by the
    Weyl constants.  Written for clarity, not speed."""
    w = params["w"]
    mask = (1 << w) - 1
    m0, m1 = params["m"]
    w0, w1 = params["k"]
    x = [int(c) & mask for c in ctr]
    k0, k1 = int(key[0]) & mask, int(key[1]) & mask
    for r in range(rounds):
        if r:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0 = m0 * x[0]
        p1 = m1 * x[2]
        hi0, lo0 = p0 >> w, p0 & mask
        hi1, lo1 = p1 >> w, p1 & mask
        x = [hi1 ^ x[1] ^ k0, lo1, hi0 ^ x[3] ^ k1, lo0]
    return x


def philox4x32(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Arguments broadcast; returns 4 uint32 arrays."""
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in (c0, c1, c2, c3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    kk0 = np.asarray(k0, dtype=np.uint64) & MASK32
    kk1 = np.asarray(k1, dtype=np.uint64) & MASK32
    m0 = np.uint64(PHILOX4x32["m"][0])
    m1 = np.uint64(PHILOX4x32["m"][1])
    w0 = np.uint64(PHILOX4x32["k"][0])
    w1 = np.uint64(PHILOX4x32["k"][1])
    s32 = np.uint64(32)
    lo = np.uint64(MASK32)
    for r in range(10):
        if r:
            kk0 = (kk0 + w0) & lo
            kk1 = (kk1 + w1) & lo
        p0 = m0 * x0
        p1 = m1 * x2
        n0 = (p1 >> s32) ^ x1 ^ kk0
        n2 = (p0 >> s32) ^ x3 ^ kk1
        x0, x1, x2, x3 = n0, p1 & lo, n2, p0 & lo
    return tuple(a.astype(np.uint32) for a in (x0, x1, x2, x3))


def seed_key(seed):
    """Philox key words (lo32, hi32) of a 64-bit row seed."""
    s = np.asarray(seed, dtype=np.uint64)
    return (s & np.uint64(MASK32)).astype(np.uint64), (s >> np.uint64(32)).astype(np.uint64)


def uniform_open01(word):
    """u = (2*(x >> 9) + 1) * 2^-24: an fp32 value in (0, 1), exact, symmetric."""
    x = np.asarray(word, dtype=np.uint32)
    odd = (x >> U32(9)).astype(np.uint32) * U32(2) + U32(1)
    return odd.astype(np.float32) * np.float32(2.0 ** -24)


def uniform_index(word, n: int):
    """floor(x * n / 2^32): a uniform integer in [0, n) from one 32-bit word."""
    x = np.asarray(word, dtype=np.uint64)
    return ((x * np.uint64(n)) >> np.uint64(32)).astype(np.int64)


def _f32c(bits: int) -> np.float32:
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


# fp32 constants by bit pattern: 1/3, 1/5, 1/7, 1/9, 1/11, sqrt(2), ln2 hi/lo.
C3, C5, C7, C9, C11 = (_f32c(b) for b in (0x3EAAAAAB, 0x3E4CCCCD, 0x3E124925,
                                          0x3DE38E39, 0x3DBA2E8C))
SQRT2 = _f32c(0x3FB504F3)
LN2_HI = _f32c(0x3F317200)   # 0.693145751953125, 15 significant bits
LN2_LO = _f32c(0x35BFBE8E)   # ln 2 - LN2_HI
ONE = np.float32(1.0)
HALF = np.float32(0.5)


def ln_f32(x):
    """Natural log of positive normal fp32 values, op-by-op in fp32."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    e = ((bits >> U32(23)) & U32(0xFF)).astype(np.int32) - 127
    m = ((bits & U32(0x7FFFFF)) | U32(0x3F800000)).view(np.float32)
    big = m > SQRT2
    m = np.where(big, m * HALF, m).astype(np.float32)
    e = e + big.astype(np.int32)
    t = (m - ONE) / (m + ONE)
    t2 = t * t
    p = C11 * t2
    p = p + C9
    p = p * t2
    p = p + C7
    p = p * t2
    p = p + C5
    p = p * t2
    p = p + C3
    p = p * t2
    p = p + ONE
    lnm = (t + t) * p
    ef = e.astype(np.float32)
    return (ef * LN2_HI + (lnm + ef * LN2_LO)).astype(np.float32)


def gumbel_f32(u):
    """G = -ln(-ln u), in fp32 with ln_f32."""
    a = -ln_f32(u)
    return (-ln_f32(a)).astype(np.float32)
