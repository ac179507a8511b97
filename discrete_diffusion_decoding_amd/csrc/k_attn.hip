// Canvas / prefix attention on MFMA for gfx950, flash-style with key splits.
//
// Mask (DiffusionGemma: causal prompt encoding, bidirectional canvas; laozijiushiniubi
// article section 2, gxsgwd news item): canvas queries see every prefix key and
// every canvas key of their own canvas; prefix queries (prefill) see keys at
// positions <= their own.  Query head h reads key/value head h / (H / Hkv).
//
// A workgroup (8 waves) owns 8 row fragments of 16 (query, head) rows that share
// one key/value head: 16 * 8 / GQ queries times the GQ query heads of that kv
// head.  Key/value tiles of 32 keys are loaded cooperatively (16-byte loads,
// clamped and branch-free) into double-buffered LDS; the next tile's loads are
// in flight while the current one is multiplied.  K rows are padded by 16 bytes
// and V^T rows (values are cached transposed, [head][dim][position]) by 16 bytes
// so the MFMA operand reads hit distinct banks.
//
// Each wave computes S^T = K Q^T with keys as the MFMA M dimension, so every
// lane holds 8 probabilities of ONE query row (keys 4*(l/16)+i and 16+4*(l/16)+i);
// those 8 values are the A operand of P V when the B operand (from V^T) uses
// the same 32-key order.  Scores are kept in log2 units.  Each key split writes
// unnormalised O with its running max / sum; attention_merge combines them.
#include <math.h>

#include "dg_kernels.hpp"

namespace dg {

template <int HD>
__global__ __launch_bounds__(512, 1) void attn_kernel(AttnArgs a) {
  constexpr int KP = HD + 8;   // K tile pitch (elements)
  constexpr int VP = 40;       // V^T tile pitch (elements): 32 keys + pad
  constexpr int KCH = 32 * HD / 8;   // 16-byte chunks of a K tile
  constexpr int VCH = HD * 4;        // 16-byte chunks of a V^T tile
  constexpr int KPT = (KCH + 511) / 512, VPT = (VCH + 511) / 512;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][32 * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][HD * VP];
  if (a.flag && *a.flag) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int GQ = a.H / a.Hkv;
  const int qpw = 128 / GQ;                      // queries per workgroup
  const int R = a.rows_per_batch;
  const int nqb = (R + qpw - 1) / qpw;
  // query blocks fastest: the blocks that read one (kv head, key split) share an XCD
  const long lb = xcd_logical_block((long)nqb * a.Hkv * a.splits * a.B);
  if (lb < 0) return;
  const int qb = (int)(lb % nqb);
  const int gy = (int)((lb / nqb) % (a.Hkv * a.splits));
  const int b = (int)(lb / ((long)nqb * a.Hkv * a.splits));
  const int g = gy % a.Hkv, split = gy / a.Hkv;
  const int q0wg = qb * qpw;
  const int hq = wave % GQ, qf = wave / GQ;      // this wave's head and query fragment
  const int h = g * GQ + hq;
  const int qrow0 = q0wg + qf * 16;
  const int lr = lane & 15, lg = lane >> 4;

  const int nk = a.n1 + a.n2;
  const int kbeg = split * a.split_len;
  int kend = min(nk, kbeg + a.split_len);
  if (a.causal) kend = min(kend, a.qpos0 + min(q0wg + qpw, R));
  const int ntile = kend > kbeg ? (kend - kbeg + 31) / 32 : 0;

  const int b1 = (a.nb1 == 1) ? 0 : b;
  const bf16_t* K1 = a.k1 + b1 * a.k1_bstride + g * a.k1_hstride;
  const bf16_t* V1 = a.vt1 + b1 * a.v1_bstride + g * a.v1_hstride;
  const bf16_t* K2 = a.k2 ? a.k2 + b * a.k2_bstride + g * a.k2_hstride : K1;
  const bf16_t* V2 = a.vt2 ? a.vt2 + b * a.v2_bstride + g * a.v2_hstride : V1;

  // Q fragments: B operand of S^T (row = lr, hd slots 32 ks + 8 lg)
  const int myq = min(qrow0 + lr, R - 1);
  const bf16_t* qp = a.q + ((long)(b * R + myq) * a.H + h) * HD + lg * 8;
  constexpr int KS = HD / 32;
  bf16x8 qfr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qfr[ks] = load_bf16x8(qp + 32 * ks);
  const int qpos = a.qpos0 + myq;
  const bool wave_live = qrow0 < R;

  // cooperative tile loads (registers -> LDS); at most two 16-byte chunks of
  // K and two of V^T per thread (hd <= 256), written out slot by slot so the
  // staging values stay in registers
  static_assert(KPT <= 2 && VPT <= 2, "tile staging assumes hd <= 256");
  uint4 ka0, ka1, va0, va1, kb0, kb1, vb0, vb1;   // two staging sets: tiles t+1 and t+2 in flight
  // Every key count here is a multiple of 32 (prefix lengths, canvases and
  // prefill chunks are), so a 32-key tile lies wholly in one source and needs
  // no clamping: its address is a wave-uniform base plus a per-thread offset
  // fixed for the whole loop.
  long koff[2], voff1[2], voff2[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + 512 * j;
    const int kc = min(c, KCH - 1), vc = min(c, VCH - 1);
    koff[j] = (long)(kc / (HD / 8)) * HD + (kc % (HD / 8)) * 8;
    voff1[j] = (long)(vc >> 2) * a.v1_pitch + (vc & 3) * 8;
    voff2[j] = (long)(vc >> 2) * a.v2_pitch + (vc & 3) * 8;
  }
#define DG_K_SRC(J) (kt_ < a.n1 ? K1 + (long)kt_ * HD : K2 + (long)(kt_ - a.n1) * HD) + koff[J]
#define DG_V_SRC(J) (kt_ < a.n1 ? V1 + kt_ + voff1[J] : V2 + (kt_ - a.n1) + voff2[J])
#define DG_ATTN_ISSUE(KT, K0, K1_, V0, V1_)                                                        \
  do {                                                                                             \
    const int kt_ = (KT);                                                                          \
    K0 = *reinterpret_cast<const uint4*>(DG_K_SRC(0));                                             \
    if (KPT > 1) K1_ = *reinterpret_cast<const uint4*>(DG_K_SRC(1));                               \
    V0 = *reinterpret_cast<const uint4*>(DG_V_SRC(0));                                             \
    if (VPT > 1) V1_ = *reinterpret_cast<const uint4*>(DG_V_SRC(1));                               \
  } while (0)
#define DG_K_PUT(BUF, C, V)                                                                        \
  do {                                                                                             \
    if (KCH % 512 == 0 || (C) < KCH)                                                               \
      *reinterpret_cast<uint4*>(&Ks[BUF][((C) / (HD / 8)) * KP + ((C) % (HD / 8)) * 8]) = (V);     \
  } while (0)
#define DG_V_PUT(BUF, KT, C, VV)                                                                   \
  do {                                                                                             \
    if (VCH % 512 == 0 || (C) < VCH)                                                               \
      *reinterpret_cast<uint4*>(&Vs[BUF][((C) >> 2) * VP + ((C) & 3) * 8]) = (VV);                  \
  } while (0)
#define DG_ATTN_STORE(BUF, KT, K0, K1_, V0, V1_)                                                   \
  do {                                                                                             \
    DG_K_PUT(BUF, tid, K0);                                                                        \
    if (KPT > 1) DG_K_PUT(BUF, tid + 512, K1_);                                                    \
    DG_V_PUT(BUF, KT, tid, V0);                                                                    \
    if (VPT > 1) DG_V_PUT(BUF, KT, tid + 512, V1_);                                                \
  } while (0)

  floatx4 O[HD / 16];
#pragma unroll
  for (int nf = 0; nf < HD / 16; ++nf) O[nf] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * 1.4426950408889634f;

  // Tile t sits in LDS buffer t & 1; the loads of tiles t+1 and t+2 are in
  // flight in the two staging sets.  Issues and stores are unconditional (tile
  // start clamped to the last tile; a store past the end fills a buffer that
  // is not read again), so the compiler's wait before each store only covers
  // the older set and nothing waits at the top of the loop.
  const int klast = kbeg + 32 * max(ntile - 1, 0);
#define DG_ATTN_TILE(BUF, KT)                                                                      \
  do {                                                                                             \
    const int kt_t_ = (KT);                                                                           \
    if (wave_live) {                                                                               \
      floatx4 s[2];                                                                                \
      _Pragma("unroll") for (int kf = 0; kf < 2; ++kf) {                                           \
        const bf16_t* kp = &Ks[BUF][(kf * 16 + lr) * KP + lg * 8];                                 \
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};                                                        \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(load_bf16x8(kp + 32 * ks), qfr[ks], acc); \
        s[kf] = acc;                                                                               \
      }                                                                                            \
      float p[8];                                                                                  \
      float mx = -INFINITY;                                                                        \
      _Pragma("unroll") for (int kf = 0; kf < 2; ++kf)                                             \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                            \
          const int key = kt_t_ + kf * 16 + lg * 4 + i;                                               \
          const bool ok = key < kend && (!a.causal || key <= qpos);                                \
          const float v = ok ? s[kf][i] * sl2 : -INFINITY;                                         \
          p[kf * 4 + i] = v;                                                                       \
          mx = fmaxf(mx, v);                                                                       \
        }                                                                                          \
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));                                                      \
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));                                                      \
      const float m_new = fmaxf(m_run, mx);                                                        \
      const bool live = m_new != -INFINITY;                                                        \
      const float alpha = live ? exp2f(m_run - m_new) : 1.0f;                                      \
      float ps = 0.f;                                                                              \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                              \
        p[e] = live ? exp2f(p[e] - m_new) : 0.f;                                                   \
        ps += p[e];                                                                                \
      }                                                                                            \
      ps += __shfl_xor(ps, 16, 64);                                                                \
      ps += __shfl_xor(ps, 32, 64);                                                                \
      l_run = l_run * alpha + ps;                                                                  \
      m_run = m_new;                                                                               \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                              \
        const float ai = __shfl(alpha, lg * 4 + i, 64);                                            \
        _Pragma("unroll") for (int nf = 0; nf < HD / 16; ++nf) O[nf][i] *= ai;                     \
      }                                                                                            \
      bf16x8 pf;                                                                                   \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) pf[e] = (__bf16)p[e];                          \
      _Pragma("unroll") for (int nf = 0; nf < HD / 16; ++nf) {                                     \
        const bf16_t* vp = &Vs[BUF][(nf * 16 + lr) * VP + lg * 4];                                 \
        const uint2 lo = *reinterpret_cast<const uint2*>(vp);                                      \
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16);                                 \
        bf16x8 vb;                                                                                 \
        vb[0] = __builtin_bit_cast(__bf16, (uint16_t)(lo.x & 0xFFFF));                             \
        vb[1] = __builtin_bit_cast(__bf16, (uint16_t)(lo.x >> 16));                                \
        vb[2] = __builtin_bit_cast(__bf16, (uint16_t)(lo.y & 0xFFFF));                             \
        vb[3] = __builtin_bit_cast(__bf16, (uint16_t)(lo.y >> 16));                                \
        vb[4] = __builtin_bit_cast(__bf16, (uint16_t)(hi.x & 0xFFFF));                             \
        vb[5] = __builtin_bit_cast(__bf16, (uint16_t)(hi.x >> 16));                                \
        vb[6] = __builtin_bit_cast(__bf16, (uint16_t)(hi.y & 0xFFFF));                             \
        vb[7] = __builtin_bit_cast(__bf16, (uint16_t)(hi.y >> 16));                                \
        O[nf] = mfma16x16x32(pf, vb, O[nf]);                                                       \
      }                                                                                            \
    }                                                                                              \
  } while (0)

  // the Q fragments are complete before the loop, so the compiler's waits
  // inside it only concern tile loads (otherwise every iteration re-waits on
  // the Q loads and drains the tile prefetch with them)
  __builtin_amdgcn_s_waitcnt(0);
  if (ntile > 0) {
    DG_ATTN_ISSUE(kbeg, ka0, ka1, va0, va1);
    DG_ATTN_ISSUE(min(kbeg + 32, klast), kb0, kb1, vb0, vb1);
    DG_ATTN_STORE(0, kbeg, ka0, ka1, va0, va1);
  }
  __syncthreads();
  for (int t = 0; t < ntile; t += 2) {
    const int kt = kbeg + 32 * t;
    // even tile t: buffer 0; set b holds tile t+1; set a takes tile t+2
    DG_ATTN_ISSUE(min(kt + 64, klast), ka0, ka1, va0, va1);
    DG_ATTN_TILE(0, kt);
    DG_ATTN_STORE(1, kt + 32, kb0, kb1, vb0, vb1);   // past the last tile: a clamped copy nobody reads
    __syncthreads();
    if (t + 1 >= ntile) break;
    // odd tile t+1: buffer 1; set a holds tile t+2; set b takes tile t+3
    DG_ATTN_ISSUE(min(kt + 96, klast), kb0, kb1, vb0, vb1);
    DG_ATTN_TILE(1, kt + 32);
    DG_ATTN_STORE(0, kt + 64, ka0, ka1, va0, va1);
    __syncthreads();
  }

#undef DG_ATTN_ISSUE
#undef DG_ATTN_TILE
#undef DG_ATTN_STORE
#undef DG_K_SRC
#undef DG_V_SRC
#undef DG_K_PUT
#undef DG_V_PUT
  if (!wave_live) return;
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
  if (a.split_len % 32 != 0 || a.rows_per_batch <= 0 || a.n1 % 32 != 0 || a.n2 % 32 != 0) return hipErrorInvalidValue;
  const int qpw = 128 / GQ;
  const long total = (long)((a.rows_per_batch + qpw - 1) / qpw) * a.Hkv * a.splits * a.B;
  if (total <= 0) return hipSuccess;
  const dim3 grid(xcd_grid(total));
  switch (a.hd) {
    case 64: hipLaunchKernelGGL(attn_kernel<64>, grid, dim3(512), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_kernel<128>, grid, dim3(512), 0, s, a); break;
    case 256: hipLaunchKernelGGL(attn_kernel<256>, grid, dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dg
