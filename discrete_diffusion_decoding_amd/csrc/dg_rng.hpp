// Counter-based random numbers for the sampler, usable on host and device.
//
// Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3" (SC'11), section 3: each round multiplies counter words 0 and 2
// by two fixed constants, keeps both halves of the 64-bit products, and mixes
// the high halves with the other two words and the key; the key advances by
// two Weyl constants between rounds.
//
// Counter layout of the denoising sampler (key = 64-bit row seed, lo word first):
//   Gumbel noise of (canvas position i, vocab entry v) at step s:
//       counter (v, i >> 2, s, 0), output word i & 3
//   re-randomised token of position i at step s: counter (i, 0, s, 1), word 0
//   initial canvas token of position i:           counter (i, 0, 0xFFFFFFFF, 1), word 0
//
// u = (2 * (x >> 9) + 1) * 2^-24 is exact in fp32 and lies in (0, 1).
// ln_dg: own fp32 natural log so GPU and CPU sampling decisions are bit-equal.
// Range reduction by the binary exponent with ln 2 split in two parts (Cody and
// Waite), mantissa folded into [sqrt(1/2), sqrt(2)), then
// ln m = 2 atanh(t) = 2 (t + t^3/3 + ... + t^11/11), t = (m-1)/(m+1), Horner in t^2.
// Each step is one IEEE fp32 operation; contraction into FMA is disabled.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define DG_HD __host__ __device__ __forceinline__
#else
#define DG_HD inline
#endif

struct dg_u32x4 { uint32_t x[4]; };

DG_HD dg_u32x4 dg_philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)M0 * c0;
    const uint64_t p1 = (uint64_t)M1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += W0;
    k1 += W1;
  }
  dg_u32x4 o;
  o.x[0] = c0; o.x[1] = c1; o.x[2] = c2; o.x[3] = c3;
  return o;
}

DG_HD float dg_bits_f32(uint32_t b) {
  union { uint32_t u; float f; } c;
  c.u = b;
  return c.f;
}

DG_HD uint32_t dg_f32_bits(float f) {
  union { uint32_t u; float f; } c;
  c.f = f;
  return c.u;
}

// (2*(x>>9)+1) * 2^-24
DG_HD float dg_uniform_open01(uint32_t x) {
  const uint32_t odd = ((x >> 9) << 1) | 1u;
  return (float)odd * dg_bits_f32(0x33800000u);  // 2^-24
}

// floor(x * n / 2^32)
DG_HD uint32_t dg_uniform_index(uint32_t x, uint32_t n) {
  return (uint32_t)(((uint64_t)x * (uint64_t)n) >> 32);
}

DG_HD float dg_ln(float x) {
#pragma clang fp contract(off)
  const uint32_t bits = dg_f32_bits(x);
  int e = (int)((bits >> 23) & 0xFFu) - 127;
  float m = dg_bits_f32((bits & 0x7FFFFFu) | 0x3F800000u);
  if (m > dg_bits_f32(0x3FB504F3u)) {  // sqrt(2)
    m = m * 0.5f;
    e += 1;
  }
  const float one = 1.0f;
  const float num = m - one;
  const float den = m + one;
  const float t = num / den;  // correctly rounded (no fast-math)
  const float t2 = t * t;
  float p = dg_bits_f32(0x3DBA2E8Cu) * t2;  // 1/11
  p = p + dg_bits_f32(0x3DE38E39u);         // 1/9
  p = p * t2;
  p = p + dg_bits_f32(0x3E124925u);         // 1/7
  p = p * t2;
  p = p + dg_bits_f32(0x3E4CCCCDu);         // 1/5
  p = p * t2;
  p = p + dg_bits_f32(0x3EAAAAABu);         // 1/3
  p = p * t2;
  p = p + one;
  const float tt = t + t;
  const float lnm = tt * p;
  const float ef = (float)e;
  const float hi = ef * dg_bits_f32(0x3F317200u);  // ln2, high 15 bits
  const float lo = ef * dg_bits_f32(0x35BFBE8Eu);  // ln2 - high part
  const float r = lnm + lo;
  return hi + r;
}

DG_HD float dg_gumbel(float u) {
#pragma clang fp contract(off)
  const float a = -dg_ln(u);
  return -dg_ln(a);
}

// 1 / tau_s in fp32, tau_s = t0 + ((t1 - t0) * s) / (S - 1) evaluated in fp64.
DG_HD float dg_inv_tau(float tau_start, float tau_end, int max_steps, int step) {
#pragma clang fp contract(off)
  const double t0 = (double)tau_start, t1 = (double)tau_end;
  double tau = t0;
  if (max_steps > 1) {
    const double num = (t1 - t0) * (double)step;
    tau = t0 + num / (double)(max_steps - 1);
  }
  return (float)(1.0 / tau);
}
