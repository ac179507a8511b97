// Canvas / prefix attention on MFMA for gfx950, flash-style with key splits.
//
// Mask (DiffusionGemma: causal prompt encoding, bidirectional canvas; laozijiushiniubi
// article section 2, gxsgwd news item): canvas queries see every prefix key and
// every canvas key of their own canvas; prefix queries (prefill) see keys at
// positions <= their own.  Query head h reads key/value head h / (H / Hkv).
//
// One wave owns 16 query rows of one head.  Per tile of 32 keys it computes
// S^T = K Q^T with keys as the MFMA M dimension, so each lane ends up holding
// 8 probabilities of ONE query row (keys 4*(l/16)+i and 16+4*(l/16)+i).  Those
// 8 values are exactly an A operand of the P V product if the same 32-key
// order is used for the B operand, which is read from V^T (values are cached
// transposed, [head][dim][position]) with two 8-byte loads.  No LDS is used.
// Scores are kept in log2 units (scale * log2 e folded in).  Each key split
// writes unnormalised O with its running max / sum; a merge kernel combines.
#include <math.h>

#include "dg_kernels.hpp"

namespace dg {

template <int HD>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  if (a.flag && *a.flag) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int GQ = a.H / a.Hkv;
  const int qb_per_wg = 4 / GQ;
  const int hq = wave % GQ, qb = wave / GQ;
  const int g = blockIdx.y % a.Hkv, split = blockIdx.y / a.Hkv;
  const int b = blockIdx.z;
  const int h = g * GQ + hq;
  const int R = a.rows_per_batch;
  const int qrow0 = (blockIdx.x * qb_per_wg + qb) * 16;
  if (qrow0 >= R) return;
  const int lr = lane & 15, lg = lane >> 4;

  const int myq = min(qrow0 + lr, R - 1);
  const bf16_t* qp = a.q + ((long)(b * R + myq) * a.H + h) * HD + lg * 8;
  constexpr int KS = HD / 32;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = load_bf16x8(qp + 32 * ks);

  const int nk = a.n1 + a.n2;
  const int kbeg = split * a.split_len;
  int kend = min(nk, kbeg + a.split_len);
  if (a.causal) kend = min(kend, a.qpos0 + min(qrow0 + 15, R - 1) + 1);
  const int qpos = a.qpos0 + myq;

  const int b1 = (a.nb1 == 1) ? 0 : b;
  const bf16_t* K1 = a.k1 + b1 * a.k1_bstride + g * a.k1_hstride;
  const bf16_t* V1 = a.vt1 + b1 * a.v1_bstride + g * a.v1_hstride;
  const bf16_t* K2 = a.k2 ? a.k2 + b * a.k2_bstride + g * a.k2_hstride : nullptr;
  const bf16_t* V2 = a.vt2 ? a.vt2 + b * a.v2_bstride + g * a.v2_hstride : nullptr;

  floatx4 O[HD / 16];
#pragma unroll
  for (int nf = 0; nf < HD / 16; ++nf) O[nf] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;

  for (int kt = kbeg; kt < kend; kt += 32) {
    floatx4 s[2];
#pragma unroll
    for (int kf = 0; kf < 2; ++kf) {
      const int key = min(kt + kf * 16 + lr, nk - 1);
      const bf16_t* kp = (key < a.n1 ? K1 + (long)key * HD : K2 + (long)(key - a.n1) * HD) + lg * 8;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(load_bf16x8(kp + 32 * ks), qf[ks], acc);
      s[kf] = acc;
    }
    float p[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kf = 0; kf < 2; ++kf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kt + kf * 16 + lg * 4 + i;
        const bool ok = key < kend && (!a.causal || key <= qpos);
        const float v = ok ? s[kf][i] * sl2 : -INFINITY;
        p[kf * 4 + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? exp2f(m_run - m_new) : 1.0f;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = live ? exp2f(p[e] - m_new) : 0.f;
      ps += p[e];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // O rows are 4*lg + i; their alpha lives in lane (4*lg + i)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, lg * 4 + i, 64);
#pragma unroll
      for (int nf = 0; nf < HD / 16; ++nf) O[nf][i] *= ai;
    }
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = (__bf16)p[e];
#pragma unroll
    for (int nf = 0; nf < HD / 16; ++nf) {
      const int dim = nf * 16 + lr;
      bf16x8 vb;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int key0 = kt + hh * 16 + lg * 4;
        uint2 raw = {0u, 0u};
        if (key0 < nk) {
          const bf16_t* vp = key0 < a.n1 ? V1 + (long)dim * a.v1_pitch + key0
                                          : V2 + (long)dim * a.v2_pitch + (key0 - a.n1);
          raw = *reinterpret_cast<const uint2*>(vp);
        }
        uint16_t w[4] = {(uint16_t)(raw.x & 0xFFFF), (uint16_t)(raw.x >> 16), (uint16_t)(raw.y & 0xFFFF),
                         (uint16_t)(raw.y >> 16)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool okk = (key0 + i) < nk;
          vb[hh * 4 + i] = __builtin_bit_cast(__bf16, okk ? w[i] : (uint16_t)0);
        }
      }
      O[nf] = mfma16x16x32(pf, vb, O[nf]);
    }
  }

  const long BR = (long)a.B * R;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = qrow0 + lg * 4 + i;
    if (row >= R) continue;
    float* op = a.opart + (((long)split * BR + (long)b * R + row) * a.H + h) * HD;
#pragma unroll
    for (int nf = 0; nf < HD / 16; ++nf) op[nf * 16 + lr] = O[nf][i];
  }
  if (lg == 0 && qrow0 + lr < R) {
    float* mp = a.mlpart + (((long)split * BR + (long)b * R + qrow0 + lr) * a.H + h) * 2;
    mp[0] = m_run;
    mp[1] = l_run;
  }
}

hipError_t attention(const AttnArgs& a, hipStream_t s) {
  const int GQ = a.H / a.Hkv;
  if (a.H % a.Hkv != 0 || (GQ != 1 && GQ != 2 && GQ != 4)) return hipErrorInvalidValue;
  if (a.split_len % 32 != 0 || a.rows_per_batch <= 0) return hipErrorInvalidValue;
  const int qb_per_wg = 4 / GQ;
  dim3 grid((a.rows_per_batch + 16 * qb_per_wg - 1) / (16 * qb_per_wg), a.Hkv * a.splits, a.B);
  switch (a.hd) {
    case 64: hipLaunchKernelGGL(attn_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(attn_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dg
