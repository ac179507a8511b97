// Row-wise kernels of one transformer layer of the denoising step (gfx950):
// embedding gather, RMSNorm (optionally folding in split-K partial sums), the
// per-step rotary table, per-head QK RMSNorm + rotary embedding writing K into
// the attention caches, the tiled V -> V^T cache scatter, split-attention merge,
// MoE router top-k, expert permutation (wavefront ballot scans) and the combine
// that also produces the next RMSNorm.  They move little data next to the
// weight streams, so they are written for latency: one workgroup per token row,
// float4 accesses, every load of a row issued before it is reduced (split and
// slot counts are template parameters, so the loops fully unroll).
#include <math.h>

#include <algorithm>

#include "dg_kernels.hpp"

namespace dg {

#define DG_MAXC4 4  // float4 columns per thread: d_model <= 4096 with 256 threads

__device__ __forceinline__ float4 f4add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 f4fma(float s, float4 a, float4 b) {
  return make_float4(s * a.x + b.x, s * a.y + b.y, s * a.z + b.z, s * a.w + b.w);
}
__device__ __forceinline__ float f4dot(float4 a) { return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w; }

__device__ __forceinline__ void store_bf16x4(bf16_t* p, float4 v) {
  uint2 o;
  o.x = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
  o.y = (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16);
  *reinterpret_cast<uint2*>(p) = o;
}
__device__ __forceinline__ float4 unpack_bf16x4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xFFFF0000u));
}
__device__ __forceinline__ float4 load_bf16x4(const bf16_t* p) {
  return unpack_bf16x4(*reinterpret_cast<const uint2*>(p));
}
// the values a bf16x4 store of v would hold
__device__ __forceinline__ float4 round_bf16x4(float4 v) {
  return make_float4(bf2f(f2bf(v.x)), bf2f(f2bf(v.y)), bf2f(f2bf(v.z)), bf2f(f2bf(v.w)));
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* tok, const bf16_t* E, int d, float* h,
                                                    const int32_t* flag) {
  if (flag && *flag) return;
  const int r = blockIdx.x;
  const bf16_t* e = E + (long)tok[r] * d;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4)
    *reinterpret_cast<float4*>(h + (long)r * d + c) = load_bf16x4(e + c);
}

hipError_t embed_rows(const int32_t* tokens, const bf16_t* E, int rows, int d, float* h, const int32_t* flag,
                      hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, s, tokens, E, d, h, flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// h += (gate ? sigmoid(gate) : 1) * sum_s part_s ; xn = bf16(rms(h) * w);
// optional router hi/lo rows (xn2 and the bf16 residual of the fp32 value).
// Every load of the row (residual, partials, gate, norm weight) is issued
// before the first store, so the row costs one memory round trip.
template <int NS>
__global__ __launch_bounds__(256) void rmsnorm_kernel(float* h, const bf16_t* w, int rows, int d, float eps,
                                                      bf16_t* out, bf16_t* split, float* dump, Partials part,
                                                      const bf16_t* pgate, const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ float red[16];
  const int r = blockIdx.x;
  const int d4 = d >> 2;
  float4* x4 = reinterpret_cast<float4*>(h + (long)r * d);
  float4 v[DG_MAXC4];
  float4 ps[DG_MAXC4][NS > 0 ? NS : 1];
  uint2 wr[DG_MAXC4], gr[DG_MAXC4];
#pragma unroll
  for (int j = 0; j < DG_MAXC4; ++j) {
    const int c4 = threadIdx.x + 256 * j;
    if (c4 < d4) {
      v[j] = x4[c4];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        ps[j][s] = reinterpret_cast<const float4*>(part.p + s * part.stride + (long)r * d)[c4];
      if (NS > 0 && pgate) gr[j] = *reinterpret_cast<const uint2*>(pgate + 4 * c4);
      wr[j] = *reinterpret_cast<const uint2*>(w + 4 * c4);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < DG_MAXC4; ++j) {
    const int c4 = threadIdx.x + 256 * j;
    if (c4 < d4) {
      if (NS > 0) {
        float4 acc = ps[j][0];
#pragma unroll
        for (int s = 1; s < NS; ++s) acc = f4add(acc, ps[j][s]);
        if (pgate) {
          const float4 gt = unpack_bf16x4(gr[j]);
          acc = make_float4(sigmoidf_(gt.x) * acc.x, sigmoidf_(gt.y) * acc.y, sigmoidf_(gt.z) * acc.z,
                            sigmoidf_(gt.w) * acc.w);
        }
        v[j] = f4add(v[j], acc);
        x4[c4] = v[j];
      }
      ss += f4dot(v[j]);
    }
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int j = 0; j < DG_MAXC4; ++j) {
    const int c4 = threadIdx.x + 256 * j;
    if (c4 < d4) {
      const float4 wv = unpack_bf16x4(wr[j]);
      const float4 y = make_float4(v[j].x * inv * wv.x, v[j].y * inv * wv.y, v[j].z * inv * wv.z,
                                   v[j].w * inv * wv.w);
      store_bf16x4(out + (long)r * d + 4 * c4, y);
      if (split) {
        store_bf16x4(split + (long)r * d + 4 * c4, y);
        const float4 hi = round_bf16x4(y);
        store_bf16x4(split + (long)(rows + r) * d + 4 * c4,
                     make_float4(y.x - hi.x, y.y - hi.y, y.z - hi.z, y.w - hi.w));
      }
      if (dump) reinterpret_cast<float4*>(dump + (long)r * d)[c4] = v[j];
    }
  }
}

hipError_t rmsnorm_rows(float* h, const bf16_t* w, int rows, int d, float eps, bf16_t* out, bf16_t* split_hi_lo,
                        float* dump, Partials part, const bf16_t* part_gate, const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d > 1024 * DG_MAXC4 || d % 4) return hipErrorInvalidValue;
#define DG_NORM_CASE(N)                                                                               \
  case N:                                                                                             \
    hipLaunchKernelGGL(rmsnorm_kernel<N>, dim3(rows), dim3(256), 0, s, h, w, rows, d, eps, out, split_hi_lo, \
                       dump, part, part_gate, flag);                                                  \
    break;
  switch (part.n) {
    DG_NORM_CASE(0) DG_NORM_CASE(1) DG_NORM_CASE(2) DG_NORM_CASE(3) DG_NORM_CASE(4)
    DG_NORM_CASE(5) DG_NORM_CASE(6) DG_NORM_CASE(7) DG_NORM_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef DG_NORM_CASE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rotary table of one pass: cos / sin of position pos0 + (r % per_batch) at
// frequency theta^(-2j/hd), computed once in fp64 for all layers of the pass.
__global__ void rope_table_kernel(float2* tab, int per_batch, int pos0, int half, float theta,
                                  const int32_t* pos_dev) {
  const int t = blockIdx.x;
  if (pos_dev) pos0 = *pos_dev;
  for (int j = threadIdx.x; j < half; j += blockDim.x) {
    const double freq = exp(-(2.0 * (double)j / (double)(2 * half)) * log((double)theta));
    double sv, cv;
    sincos((double)(pos0 + t) * freq, &sv, &cv);
    tab[(long)t * half + j] = make_float2((float)cv, (float)sv);
  }
}

hipError_t rope_table(float2* tab, int per_batch, int pos0, int hd, float theta, const int32_t* pos_dev,
                      hipStream_t s) {
  if (per_batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3(per_batch), dim3(128), 0, s, tab, per_batch, pos0, hd / 2, theta,
                     pos_dev);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// sum over the wave, in every lane: lane pairs (xor 1, xor 2), mirrored
// halves of 8 and 16 lanes, then the gfx950 row swaps of 16 and 32 lanes
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x140, 0xF, 0xF, false));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// One wave per (token row, head): q heads, then k heads.  RMSNorm over
// head_dim, then rotate-half RoPE from the table.  Lane l holds the EPL =
// hd/64 consecutive elements EPL*l ..; the rotary partner of element e is
// e +- hd/2, held by lane l ^ 32 in the same position.
template <int HD>
__device__ __forceinline__ void qk_rope_head(const QkRopeArgs& a, int r, int hh) {
  constexpr int HALF = HD / 2;
  constexpr int EPL = HD / 64;
  const int tloc = r % a.per_batch, bidx = r / a.per_batch;
  const int lane = threadIdx.x & 63;
  const int e0 = EPL * lane;
  const int qkvd = (a.H + 2 * a.Hkv) * HD;
  const bool isq = hh < a.H;
  const bf16_t* xs = a.qkv + (long)r * qkvd + hh * HD + e0;
  const bf16_t* nw = (isq ? a.qnorm : a.knorm) + e0;
  const float2* tab = a.rope + (long)tloc * HALF + (e0 < HALF ? e0 : e0 - HALF);
  float x[EPL], w[EPL];
  float2 cs[EPL];
  static_assert(EPL == 1 || EPL == 2 || EPL == 4, "head_dim 64, 128 or 256");
  if constexpr (EPL == 4) {   // 8-byte element loads, 16-byte table loads
    const uint2 xv = *reinterpret_cast<const uint2*>(xs);
    const uint2 wv = *reinterpret_cast<const uint2*>(nw);
    const float4 t0 = *reinterpret_cast<const float4*>(tab);
    const float4 t1 = *reinterpret_cast<const float4*>(tab + 2);
    x[0] = bf2f(xv.x & 0xFFFF); x[1] = bf2f(xv.x >> 16); x[2] = bf2f(xv.y & 0xFFFF); x[3] = bf2f(xv.y >> 16);
    w[0] = bf2f(wv.x & 0xFFFF); w[1] = bf2f(wv.x >> 16); w[2] = bf2f(wv.y & 0xFFFF); w[3] = bf2f(wv.y >> 16);
    cs[0] = make_float2(t0.x, t0.y); cs[1] = make_float2(t0.z, t0.w);
    cs[2] = make_float2(t1.x, t1.y); cs[3] = make_float2(t1.z, t1.w);
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      x[j] = bf2f(xs[j]);
      w[j] = bf2f(nw[j]);
      cs[j] = tab[j];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) ss += x[j] * x[j];
  ss = wave_sum_dpp(ss);
  const float inv = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
  for (int j = 0; j < EPL; ++j) x[j] = x[j] * inv * w[j];
  const float sgn = e0 < HALF ? -1.f : 1.f;
  bf16_t* dst = isq ? a.q + ((long)r * a.H + hh) * HD + e0
                    : a.kdst + bidx * a.k_bstride + (hh - a.H) * a.k_hstride + (long)((a.pos_dev ? *a.pos_dev : a.t_offset) + tloc) * HD + e0;
  uint16_t y[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]), __float_as_uint(x[j]), false, false);
    // lanes < 32 get the partner from swap output 1, lanes >= 32 from output 0
    const float partner = __uint_as_float(lane < 32 ? sw[1] : sw[0]);
    y[j] = f2bf(x[j] * cs[j].x + sgn * partner * cs[j].y);
  }
  if constexpr (EPL == 4) {
    *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)y[0] | ((uint32_t)y[1] << 16), (uint32_t)y[2] | ((uint32_t)y[3] << 16));
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) dst[j] = y[j];
  }
}

// V^T scatter: a workgroup moves 32 positions x 64 dims of one kv head through
// LDS (one 16-byte load per thread), then each thread writes 8 positions of
// one dim as a 16-byte store.  The V^T caches are tile-major: position p of
// dim d sits at ((p / 32) hd + d) 32 + p % 32, so a 32-key tile is one
// contiguous block.  The LDS row pitch of 66 values staggers the banks of the
// 8-row steps read together.
constexpr int kVtPitch = 66;
template <int HD>
__device__ __forceinline__ void vt_scatter_block(const QkRopeArgs& a, int g, int t0, int d0, bf16_t* tile) {
  const int tid = threadIdx.x;
  const int qkvd = (a.H + 2 * a.Hkv) * HD;
  {
    const int tr = tid >> 3, c = (tid & 7) * 8;
    const int r = min(t0 + tr, a.rows - 1);
    const uint4 v = *reinterpret_cast<const uint4*>(a.qkv + (long)r * qkvd + (a.H + a.Hkv + g) * HD + d0 + c);
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + tr * kVtPitch + c);   // 4-byte aligned (even pitch)
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  }
  __syncthreads();
  const int bidx = t0 / a.per_batch, p0 = (a.pos_dev ? *a.pos_dev : a.t_offset) + t0 % a.per_batch;
  const int dim = tid >> 2, pg = (tid & 3) * 8;
  const int nval = min(32, a.rows - t0);
  bf16_t* vt = a.vtdst + bidx * a.v_bstride + g * a.v_hstride + (long)(d0 + dim) * 32;
  uint16_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = tile[(pg + i) * kVtPitch + dim];
  const int p = p0 + pg;
  if (pg + 8 <= nval && (p0 & 7) == 0) {   // 8 positions inside one tile
    *reinterpret_cast<uint4*>(vt + (long)(p >> 5) * (32 * HD) + (p & 31)) =
        make_uint4((uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
                   (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16));
  } else {
    for (int i = 0; i < 8 && pg + i < nval; ++i) vt[(long)((p + i) >> 5) * (32 * HD) + ((p + i) & 31)] = v[i];
  }
}

// one launch of 4-wave blocks: V^T blocks (32 positions x 64 dims of one kv
// head) first, then blocks of 4 waves, each wave the norm + RoPE of one
// (row, q / k head)
template <int HD>
__global__ __launch_bounds__(256) void qk_rope_kernel(QkRopeArgs a) {
  if (a.flag && *a.flag) return;
  __shared__ __attribute__((aligned(16))) bf16_t tile[32 * kVtPitch];
  const int nh = a.H + a.Hkv;
  const int nt = (a.rows + 31) / 32, nd = HD / 64;
  const int nvt = nt * nd * a.Hkv;
  const int bx = blockIdx.x;
  if (bx < nvt) {
    vt_scatter_block<HD>(a, bx / (nt * nd), ((bx / nd) % nt) * 32, (bx % nd) * 64, tile);
  } else {
    const int u = (bx - nvt) * 4 + (int)(threadIdx.x >> 6);
    if (u < a.rows * nh) qk_rope_head<HD>(a, u / nh, u % nh);
  }
}

hipError_t qk_norm_rope(const QkRopeArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.per_batch % 32 != 0 && a.per_batch != a.rows) return hipErrorInvalidValue;
  const long nvt = (long)((a.rows + 31) / 32) * (a.hd / 64) * a.Hkv;
  const dim3 grid((unsigned)(nvt + ((long)a.rows * (a.H + a.Hkv) + 3) / 4));
  switch (a.hd) {
    case 64: hipLaunchKernelGGL(qk_rope_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(qk_rope_kernel<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(qk_rope_kernel<256>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge of key-split attention partials (scores kept in log2 units): block
// (r, y) takes heads y hpb .. y hpb + hpb - 1 of row r; the split weights
// 2^(m_s - M) / L of its heads are formed once in LDS, then each thread sums
// its float4 columns over the splits.  The partial outputs do not depend on
// the weights, so a thread's first kMergeAhead columns are loaded before the
// (m, l) pairs are read: the block costs one memory round trip, not one per
// column pass.  Few rows (decoding) take 1024 / hd heads per block, so that a
// thread makes one pass; many rows take every head.
constexpr int kMergeAhead = 4;
template <int NSP>
__global__ __launch_bounds__(256) void attn_merge_kernel(const bf16_t* op, const float* ml, int rows, int H, int hd,
                                                         int hpb, bf16_t* out, const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ float wts[64 * NSP];
  const int r = blockIdx.x;
  const int h0 = blockIdx.y * hpb, h1 = min(H, h0 + hpb);
  const long srow = (long)rows * H;
  const long rowoff = (long)r * H * hd;
  const long sstride = srow * hd;
  const int i0 = h0 * hd / 4 + (int)threadIdx.x, n4 = h1 * hd / 4;
  uint2 pre[kMergeAhead][NSP];
#pragma unroll
  for (int g = 0; g < kMergeAhead; ++g) {
    const int i4 = i0 + 256 * g;
    if (i4 < n4) {
#pragma unroll
      for (int s = 0; s < NSP; ++s) pre[g][s] = *reinterpret_cast<const uint2*>(op + s * sstride + rowoff + 4 * i4);
    }
  }
  for (int h = h0 + threadIdx.x; h < h1; h += 256) {
    const long base = (long)r * H + h;
    float mv[NSP], lv[NSP];
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NSP; ++s) {
      mv[s] = ml[(s * srow + base) * 2];
      lv[s] = ml[(s * srow + base) * 2 + 1];
      M = fmaxf(M, mv[s]);
    }
    // split s holds O_s / l_s; its weight in the merged softmax is l_s 2^(m_s - M) / L
    float L = 0.f;
#pragma unroll
    for (int s = 0; s < NSP; ++s) {
      mv[s] = (mv[s] == -INFINITY) ? 0.f : exp2f(mv[s] - M) * lv[s];
      L += mv[s];
    }
    const float il = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
    for (int s = 0; s < NSP; ++s) wts[h * NSP + s] = mv[s] * il;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < kMergeAhead; ++g) {
    const int i4 = i0 + 256 * g;
    if (i4 < n4) {
      const int h = (4 * i4) / hd;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int s = 0; s < NSP; ++s) acc = f4fma(wts[h * NSP + s], unpack_bf16x4(pre[g][s]), acc);
      store_bf16x4(out + rowoff + 4 * i4, acc);
    }
  }
  for (int i4 = i0 + 256 * kMergeAhead; i4 < n4; i4 += 256) {
    const int h = (4 * i4) / hd;
    float4 vals[NSP];
#pragma unroll
    for (int s = 0; s < NSP; ++s) vals[s] = load_bf16x4(op + s * sstride + rowoff + 4 * i4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < NSP; ++s) acc = f4fma(wts[h * NSP + s], vals[s], acc);
    store_bf16x4(out + rowoff + 4 * i4, acc);
  }
}

hipError_t attention_merge(const bf16_t* opart, const float* mlpart, int splits, int rows, int H, int hd,
                           bf16_t* out, const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (H > 64 || hd % 4) return hipErrorInvalidValue;
  const int hpb = rows < 64 ? std::max(1, 1024 / hd) : H;
  const dim3 grid(rows, (H + hpb - 1) / hpb);
#define DG_MERGE_CASE(N)                                                                               \
  case N:                                                                                              \
    hipLaunchKernelGGL(attn_merge_kernel<N>, grid, dim3(256), 0, s, opart, mlpart, rows, H, hd, hpb, out, flag); \
    break;
  switch (splits) {
    DG_MERGE_CASE(1) DG_MERGE_CASE(2) DG_MERGE_CASE(3) DG_MERGE_CASE(4) DG_MERGE_CASE(5) DG_MERGE_CASE(6)
    DG_MERGE_CASE(7) DG_MERGE_CASE(8) DG_MERGE_CASE(9) DG_MERGE_CASE(10) DG_MERGE_CASE(11) DG_MERGE_CASE(12)
    DG_MERGE_CASE(13) DG_MERGE_CASE(14) DG_MERGE_CASE(15) DG_MERGE_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef DG_MERGE_CASE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router top-k: logits = hi-part + lo-part products (an fp32-accurate product
// from two bf16 MFMA passes) summed over the split-K partials, the k largest (ties to the lower expert index, as a stable sort of the
// negated logits), gates = softmax over the k selected logits.  One wave per
// token row: each lane holds experts lane + 64 j as 64-bit keys (order-
// preserving bits of the logit, then the complemented index), and k rounds of
// a wave-wide maximum pick the experts in order.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(0xFFFF - e);
}
__device__ __forceinline__ float topk_key_value(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
template <int CTRL>
__device__ __forceinline__ uint64_t umax64_dpp(uint64_t x) {
  const int lo = (int)(uint32_t)x, hi = (int)(uint32_t)(x >> 32);
  const uint32_t lo2 = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  const uint32_t hi2 = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
  const uint64_t y = ((uint64_t)hi2 << 32) | lo2;
  return x > y ? x : y;
}
template <bool W32>
__device__ __forceinline__ uint64_t umax64_swap(uint64_t x) {
  const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  auto l = W32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false) : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto h = W32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false) : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const uint64_t a = ((uint64_t)h[0] << 32) | l[0], b = ((uint64_t)h[1] << 32) | l[1];
  return a > b ? a : b;
}
// maximum over the wave, in every lane: lane pairs (xor 1, xor 2), mirrored
// halves of 8 and 16 lanes, then the row swaps of 16 and 32 lanes
__device__ __forceinline__ uint64_t wave_umax64(uint64_t x) {
  x = umax64_dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  x = umax64_dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  x = umax64_dpp<0x141>(x);   // row_half_mirror
  x = umax64_dpp<0x140>(x);   // row_mirror
  x = umax64_swap<false>(x);
  return umax64_swap<true>(x);
}

// Row r's slots: its NK routed experts (gates: softmax over their logits),
// then ns always-on experts E .. E + ns - 1 with gate 1 (the shared FFN's
// blocks, when they run as experts); the dumps hold the routed ones only.
// One wave per row; sidx (may be null) takes a copy of the row's slots.
template <int NS, int NK>
__device__ __forceinline__ void topk_wave_row(const Partials& rl, int rows, int E, int ns, int r, int32_t* idx,
                                              float* gate, int32_t* idx_dump, float* gate_dump, float* logit_dump,
                                              int32_t* sidx) {
  const int lane = threadIdx.x & 63;
  // every partial of the row is loaded before the first (dump) store
  float hp[4][NS], lp[4][NS];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (64 * j < E && e < E) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        hp[j][s] = rl.p[s * rl.stride + (long)r * E + e];
        lp[j][s] = rl.p[s * rl.stride + (long)(rows + r) * E + e];
      }
    }
  }
  uint64_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    key[j] = 0;
    const int e = lane + 64 * j;
    if (64 * j < E && e < E) {
      float h = 0.f, l = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        h += hp[j][s];
        l += lp[j][s];
      }
      key[j] = topk_key(h + l, e);
      if (logit_dump) logit_dump[(long)r * E + e] = h + l;
    }
  }
  float mine_v = 0.f, top_v = 0.f;
  int mine_e = 0;
#pragma unroll
  for (int t = 0; t < NK; ++t) {
    const uint64_t best = wave_umax64(max(max(key[0], key[1]), max(key[2], key[3])));
    const int e = 0xFFFF - (int)(best & 0xFFFF);
    const float v = topk_key_value(best);
    if (t == 0) top_v = v;
    if (lane == t) {
      mine_v = v;
      mine_e = e;
    }
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((e >> 6) == j) key[j] = 0;
    }
  }
  // softmax over the selected logits (lane t holds selection t)
  float ex = lane < NK ? expf(mine_v - top_v) : 0.f;
  float den = ex;
#pragma unroll
  for (int o = 1; o < NK; o <<= 1) den += __shfl_xor(den, o, 64);
  const int ko = NK + ns;
  if (lane < NK) {
    const float gt = ex / den;
    idx[(long)r * ko + lane] = mine_e;
    gate[(long)r * ko + lane] = gt;
    if (sidx) sidx[r * ko + lane] = mine_e;
    if (idx_dump) idx_dump[(long)r * NK + lane] = mine_e;
    if (gate_dump) gate_dump[(long)r * NK + lane] = gt;
  } else if (lane < ko) {
    idx[(long)r * ko + lane] = E + lane - NK;
    gate[(long)r * ko + lane] = 1.f;
    if (sidx) sidx[r * ko + lane] = E + lane - NK;
  }
}

template <int NS, int NK>
__global__ __launch_bounds__(64) void topk_kernel(Partials rl, int rows, int E, int ns, int32_t* idx, float* gate,
                                                  int32_t* idx_dump, float* gate_dump, float* logit_dump,
                                                  const int32_t* flag) {
  if (flag && *flag) return;
  topk_wave_row<NS, NK>(rl, rows, E, ns, blockIdx.x, idx, gate, idx_dump, gate_dump, logit_dump, nullptr);
}

hipError_t router_topk(Partials rlog, int rows, int E, int k, int ns, int32_t* idx, float* gate, int32_t* idx_dump,
                       float* gate_dump, float* logit_dump, const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (E > 256 || k > E || ns < 0 || k + ns > 64 || rlog.n < 1 || rlog.n > 8) return hipErrorInvalidValue;
  const dim3 grid(rows), block(64);
#define DG_TOPK_NS(NK)                                                                                   \
  switch (rlog.n) {                                                                                      \
    case 1: hipLaunchKernelGGL((topk_kernel<1, NK>), grid, block, 0, s, rlog, rows, E, ns, idx, gate, idx_dump, gate_dump, logit_dump, flag); break; \
    case 2: hipLaunchKernelGGL((topk_kernel<2, NK>), grid, block, 0, s, rlog, rows, E, ns, idx, gate, idx_dump, gate_dump, logit_dump, flag); break; \
    case 3: hipLaunchKernelGGL((topk_kernel<3, NK>), grid, block, 0, s, rlog, rows, E, ns, idx, gate, idx_dump, gate_dump, logit_dump, flag); break; \
    case 4: hipLaunchKernelGGL((topk_kernel<4, NK>), grid, block, 0, s, rlog, rows, E, ns, idx, gate, idx_dump, gate_dump, logit_dump, flag); break; \
    case 5: hipLaunchKernelGGL((topk_kernel<5, NK>), grid, block, 0, s, rlog, rows, E, ns, idx, gate, idx_dump, gate_dump, logit_dump, flag); break; \
    case 6: hipLaunchKernelGGL((topk_kernel<6, NK>), grid, block, 0, s, rlog, rows, E, ns, idx, gate, idx_dump, gate_dump, logit_dump, flag); break; \
    case 7: hipLaunchKernelGGL((topk_kernel<7, NK>), grid, block, 0, s, rlog, rows, E, ns, idx, gate, idx_dump, gate_dump, logit_dump, flag); break; \
    default: hipLaunchKernelGGL((topk_kernel<8, NK>), grid, block, 0, s, rlog, rows, E, ns, idx, gate, idx_dump, gate_dump, logit_dump, flag); break; \
  }
  switch (k) {
    case 1: DG_TOPK_NS(1) break;
    case 2: DG_TOPK_NS(2) break;
    case 4: DG_TOPK_NS(4) break;
    case 8: DG_TOPK_NS(8) break;
    default: return hipErrorInvalidValue;
  }
#undef DG_TOPK_NS
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Expert permutation in one workgroup of NT threads.
// Assignment a = row * k + j takes position p in its expert e from an LDS
// counter (atomic add; the order of rows within an expert is arbitrary and
// changes no result: every row of an expert GEMM depends on its own
// activation row only, and the combine reads the k slots of a row in j
// order), then goes to slot offsets[e] + p.  Assignments are taken in chunks
// of kPermPB per thread whose loads are issued together (one memory round
// trip per chunk); the first chunk's experts and positions stay in
// registers, later chunks park p in slot_of[a] (this thread's own write)
// until the offsets are known.
constexpr int kPermPB = 8;
template <int NT>
__device__ __forceinline__ void permute_body(const int32_t* idx, int na, int k, int E, int32_t* counts,
                                             int32_t* offsets, int32_t* slot_of, int32_t* slot_row, int4* items,
                                             int32_t* n_items, int chunk) {
  __shared__ int cnt[256];
  __shared__ int off[257];
  __shared__ int ibase[257];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int CH = kPermPB * NT;
  int e0[kPermPB], p0[kPermPB];
#pragma unroll
  for (int j = 0; j < kPermPB; ++j) {
    const int a = tid + NT * j;
    e0[j] = a < na ? idx[a] : 0;
  }
  if (tid < 256) cnt[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPermPB; ++j) {
    const int a = tid + NT * j;
    p0[j] = a < na ? atomicAdd(&cnt[e0[j]], 1) : 0;
  }
  for (int a0 = CH; a0 < na; a0 += CH) {
    int ev[kPermPB];
#pragma unroll
    for (int j = 0; j < kPermPB; ++j) {
      const int a = a0 + tid + NT * j;
      ev[j] = a < na ? idx[a] : 0;
    }
#pragma unroll
    for (int j = 0; j < kPermPB; ++j) {
      const int a = a0 + tid + NT * j;
      if (a < na) slot_of[a] = atomicAdd(&cnt[ev[j]], 1);
    }
  }
  __syncthreads();
  // exclusive scans over the experts of the row counts and of the item counts:
  // waves 0-3 scan 64 experts each (shuffle scan), then add the wave totals
  __shared__ int wtot[4][2];
  int c = 0, ni = 0, ic = 0, ii = 0;
  if (tid < 256) {
    c = tid < E ? cnt[tid] : 0;
    ni = (c + chunk - 1) / chunk;
    ic = c;
    ii = ni;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int uc = __shfl_up(ic, o, 64), ui = __shfl_up(ii, o, 64);
      if (lane >= o) {
        ic += uc;
        ii += ui;
      }
    }
    if (lane == 63) {
      wtot[wave][0] = ic;
      wtot[wave][1] = ii;
    }
  }
  __syncthreads();
  if (tid < 256) {
    for (int w = 0; w < wave; ++w) {
      ic += wtot[w][0];
      ii += wtot[w][1];
    }
    if (tid < E) {
      off[tid] = ic - c;
      ibase[tid] = ii - ni;
    }
    if (tid == E - 1) {
      off[E] = ic;
      ibase[E] = ii;
      *n_items = ii;
    }
  }
  __syncthreads();
  for (int e = tid; e <= E; e += NT) {
    offsets[e] = off[e];
    if (e < E) {
      counts[e] = cnt[e];
      int i = ibase[e];
      const int nc = (cnt[e] + chunk - 1) / chunk;
      for (int r = 0, c = 0; r < cnt[e]; r += chunk, ++i, ++c)
        items[i] = make_int4(e, off[e] + r, min(chunk, cnt[e] - r), (c << 16) | nc);
    }
  }
#pragma unroll
  for (int j = 0; j < kPermPB; ++j) {
    const int a = tid + NT * j;
    if (a < na) {
      const int slot = off[e0[j]] + p0[j];
      slot_of[a] = slot;
      slot_row[slot] = a / k;
    }
  }
  for (int a0 = CH; a0 < na; a0 += CH) {
    int ev[kPermPB], pv[kPermPB];
#pragma unroll
    for (int j = 0; j < kPermPB; ++j) {
      const int a = a0 + tid + NT * j;
      ev[j] = a < na ? idx[a] : 0;
      pv[j] = a < na ? slot_of[a] : 0;
    }
#pragma unroll
    for (int j = 0; j < kPermPB; ++j) {
      const int a = a0 + tid + NT * j;
      if (a < na) {
        const int slot = off[ev[j]] + pv[j];
        slot_of[a] = slot;
        slot_row[slot] = a / k;
      }
    }
  }
}

__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* idx, int na, int k, int E, int32_t* counts,
                                                       int32_t* offsets, int32_t* slot_of, int32_t* slot_row,
                                                       int4* items, int32_t* n_items, int chunk,
                                                       const int32_t* flag) {
  if (flag && *flag) return;
  permute_body<1024>(idx, na, k, E, counts, offsets, slot_of, slot_row, items, n_items, chunk);
}

// Few rows (decoding, at most 4): the top-k of row r (wave r, as topk_kernel)
// and the expert permutation (as permute_kernel, over the slots in LDS) in one
// workgroup, one launch instead of two.
template <int NS, int NK>
__global__ __launch_bounds__(256) void topk_permute_kernel(Partials rl, int rows, int E, int ns, int32_t* idx,
                                                           float* gate, int32_t* idx_dump, float* gate_dump,
                                                           float* logit_dump, int32_t* counts, int32_t* offsets, int32_t* slot_of,
                                                           int32_t* slot_row, int4* items, int32_t* n_items,
                                                           int chunk, const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ int32_t sidx[4 * 64];
  const int r = threadIdx.x >> 6;
  const int ko = NK + ns;
  if (r < rows) topk_wave_row<NS, NK>(rl, rows, E, ns, r, idx, gate, idx_dump, gate_dump, logit_dump, sidx);
  __syncthreads();
  permute_body<256>(sidx, rows * ko, ko, E + ns, counts, offsets, slot_of, slot_row, items, n_items, chunk);
}

hipError_t router_topk_permute(Partials rlog, int rows, int E, int k, int ns, int32_t* idx, float* gate,
                               int32_t* idx_dump, float* gate_dump, float* logit_dump, int32_t* counts, int32_t* offsets,
                               int32_t* slot_of, int32_t* slot_row, int4* items, int32_t* n_items, int chunk,
                               const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rows > 4 || E > 256 || k > E || ns < 0 || k + ns > 64 || E + ns > 255 || chunk < 1 || rlog.n < 1 ||
      rlog.n > 8)
    return hipErrorInvalidValue;
#define DG_TP(NS_, NK_)                                                                                       \
  hipLaunchKernelGGL((topk_permute_kernel<NS_, NK_>), dim3(1), dim3(256), 0, s, rlog, rows, E, ns, idx, gate, \
                     idx_dump, gate_dump, logit_dump, counts, offsets, slot_of, slot_row, items, n_items, chunk, flag)
#define DG_TP_NS(NK_)                       \
  switch (rlog.n) {                         \
    case 1: DG_TP(1, NK_); break;           \
    case 2: DG_TP(2, NK_); break;           \
    case 3: DG_TP(3, NK_); break;           \
    case 4: DG_TP(4, NK_); break;           \
    case 5: DG_TP(5, NK_); break;           \
    case 6: DG_TP(6, NK_); break;           \
    case 7: DG_TP(7, NK_); break;           \
    default: DG_TP(8, NK_); break;          \
  }
  switch (k) {
    case 1: DG_TP_NS(1) break;
    case 2: DG_TP_NS(2) break;
    case 4: DG_TP_NS(4) break;
    case 8: DG_TP_NS(8) break;
    default: return hipErrorInvalidValue;
  }
#undef DG_TP_NS
#undef DG_TP
  return hipGetLastError();
}

hipError_t moe_permute(const int32_t* idx, int rows, int k, int E, int32_t* counts, int32_t* offsets,
                       int32_t* slot_of, int32_t* slot_row, int4* items, int32_t* n_items, int chunk,
                       const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (E > 255 || chunk < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), 0, s, idx, rows * k, k, E, counts, offsets, slot_of,
                     slot_row, items, n_items, chunk, flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// h[r] += sum_s ys_s[r] + sum_j gate[r,j] * Y[slot[r,j]] (expert outputs Y in bf16,
// as stored by the down projection), then the next RMSNorm.  Two memory round
// trips per row: the slots and gates, then every other load of the row
// (expert rows, shared partials, residual, next norm weight) before the
// first store.
template <int NS, int NK>
__global__ __launch_bounds__(256) void combine_kernel(float* h, Partials ys, const bf16_t* Y,
                                                      const int32_t* slot_of, const float* gate, int d,
                                                      const bf16_t* nw, float eps, bf16_t* xn, float* dump,
                                                      const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ float red[16];
  const int r = blockIdx.x;
  const int d4 = d >> 2;
  int sl[NK];
  float gt[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    sl[j] = slot_of[(long)r * NK + j];
    gt[j] = gate[(long)r * NK + j];
  }
  float4* x4 = reinterpret_cast<float4*>(h + (long)r * d);
  float4 v[DG_MAXC4];
  uint2 yr[DG_MAXC4][NK], wr[DG_MAXC4];
  float4 pv[DG_MAXC4][NS > 0 ? NS : 1];
#pragma unroll
  for (int c = 0; c < DG_MAXC4; ++c) {
    const int c4 = threadIdx.x + 256 * c;
    if (c4 < d4) {
#pragma unroll
      for (int j = 0; j < NK; ++j) yr[c][j] = *reinterpret_cast<const uint2*>(Y + (long)sl[j] * d + 4 * c4);
#pragma unroll
      for (int s = 0; s < NS; ++s) pv[c][s] = reinterpret_cast<const float4*>(ys.p + s * ys.stride + (long)r * d)[c4];
      v[c] = x4[c4];
      if (nw) wr[c] = *reinterpret_cast<const uint2*>(nw + 4 * c4);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < DG_MAXC4; ++c) {
    const int c4 = threadIdx.x + 256 * c;
    if (c4 < d4) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < NK; ++j) acc = f4fma(gt[j], unpack_bf16x4(yr[c][j]), acc);
#pragma unroll
      for (int s = 0; s < NS; ++s) acc = f4add(acc, pv[c][s]);
      v[c] = f4add(v[c], acc);
      x4[c4] = v[c];
      ss += f4dot(v[c]);
    }
  }
  if (!nw && !dump) return;
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int c = 0; c < DG_MAXC4; ++c) {
    const int c4 = threadIdx.x + 256 * c;
    if (c4 < d4) {
      if (nw) {
        const float4 wv = unpack_bf16x4(wr[c]);
        store_bf16x4(xn + (long)r * d + 4 * c4, make_float4(v[c].x * inv * wv.x, v[c].y * inv * wv.y,
                                                            v[c].z * inv * wv.z, v[c].w * inv * wv.w));
      }
      if (dump) reinterpret_cast<float4*>(dump + (long)r * d)[c4] = v[c];
    }
  }
}

template <int NK>
static hipError_t combine_k(float* h, Partials ys, const bf16_t* Y, const int32_t* slot_of, const float* gate,
                            int rows, int d, const bf16_t* nw, float eps, bf16_t* xn, float* dump,
                            const int32_t* flag, hipStream_t s) {
#define DG_COMB_CASE(N)                                                                                   \
  case N:                                                                                                 \
    hipLaunchKernelGGL((combine_kernel<N, NK>), dim3(rows), dim3(256), 0, s, h, ys, Y, slot_of, gate, d, nw, eps, \
                       xn, dump, flag);                                                                   \
    break;
  switch (ys.n) {
    DG_COMB_CASE(0) DG_COMB_CASE(1) DG_COMB_CASE(2) DG_COMB_CASE(3) DG_COMB_CASE(4)
    DG_COMB_CASE(5) DG_COMB_CASE(6) DG_COMB_CASE(7) DG_COMB_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef DG_COMB_CASE
  return hipGetLastError();
}

hipError_t moe_combine(float* h, Partials ys, const bf16_t* Y, const int32_t* slot_of, const float* gate, int rows,
                       int d, int k, const bf16_t* next_w, float eps, bf16_t* xn, float* dump, const int32_t* flag,
                       hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d > 1024 * DG_MAXC4 || d % 4) return hipErrorInvalidValue;
  switch (k) {
    case 1: return combine_k<1>(h, ys, Y, slot_of, gate, rows, d, next_w, eps, xn, dump, flag, s);
    case 2: return combine_k<2>(h, ys, Y, slot_of, gate, rows, d, next_w, eps, xn, dump, flag, s);
    case 4: return combine_k<4>(h, ys, Y, slot_of, gate, rows, d, next_w, eps, xn, dump, flag, s);
    case 8: return combine_k<8>(h, ys, Y, slot_of, gate, rows, d, next_w, eps, xn, dump, flag, s);
    case 11: return combine_k<11>(h, ys, Y, slot_of, gate, rows, d, next_w, eps, xn, dump, flag, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t* p, int32_t v, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void fill_u16_kernel(uint16_t* p, uint16_t v, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t fill_i32(int32_t* p, int32_t v, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}
hipError_t fill_u16(uint16_t* p, uint16_t v, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace dg
