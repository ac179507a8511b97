// Sampler of the denoising step (gfx950): per-position entropy, Gumbel-max
// sample, argmax, entropy lock, re-randomisation of unlocked positions and the
// adaptive stop (laozijiushiniubi article section 4; multinomial noise and
// editable locked tokens, section 1), plus the softmax probabilities used by
// the self-conditioning soft-prediction embedding (section 2).
//
// sample_partial: one workgroup per (4 canvas positions, vocab slice).  The
// four positions share every Philox block: block (v, i >> 2, s, 0) gives word
// i & 3 to position i, so one 10-round Philox call feeds four Gumbel scores.
// Each thread keeps an online (max, sum exp, sum exp * shifted logit) triple,
// the argmax and the best Gumbel score; the workgroup reduces them per position.
// sample_finish: one workgroup per canvas row merges the slices in vocab order
// (ties -> lowest index), takes the lock / stop decisions and writes tokens.
#include <math.h>

#include "dg_kernels.hpp"
#include "dg_rng.hpp"

namespace dg {

struct Stat {
  float m, Z, A;   // max logit, sum e^(l-m), sum e^(l-m)(l-m)
  float av; int ai;  // argmax
  float gv; int gi;  // best Gumbel score
};

__device__ __forceinline__ void stat_merge(Stat& x, const Stat& y) {
  if (y.m != -INFINITY) {
    if (x.m == -INFINITY) {
      x.m = y.m; x.Z = y.Z; x.A = y.A;
    } else {
      const float M = fmaxf(x.m, y.m);
      const float fx = __expf(x.m - M), fy = __expf(y.m - M);
      x.A = fx * (x.A + (x.m - M) * x.Z) + fy * (y.A + (y.m - M) * y.Z);
      x.Z = fx * x.Z + fy * y.Z;
      x.m = M;
    }
  }
  if (y.av > x.av || (y.av == x.av && y.ai < x.ai)) { x.av = y.av; x.ai = y.ai; }
  if (y.gv > x.gv || (y.gv == x.gv && y.gi < x.gi)) { x.gv = y.gv; x.gi = y.gi; }
}

__device__ __forceinline__ int row_step(const SampleArgs& a, int b) {
  return a.step_arg >= 0 ? a.step_arg : a.steps[b];
}

// Gumbel noise through the hardware log2: over all 2^23 uniforms that
// dg_uniform_open01 can produce it differs from dg_gumbel by at most 1.6e-6
// (measured exhaustively on gfx950), so kGumbelScreen bounds the difference.
// It screens candidates; decisions are taken on dg_gumbel only.
constexpr float kGumbelScreen = 4e-6f;
__device__ __forceinline__ float gumbel_screen(float u) {
  const float LN2 = 0.693147180559945f;
  return -LN2 * __builtin_amdgcn_logf(-LN2 * __builtin_amdgcn_logf(u));
}
// scaled logit and score: separate IEEE operations (no contraction), shared by
// the screen and the exact score so that they differ only through the noise
__device__ __forceinline__ float scale_logit(float l, float inv_tau) {
#pragma clang fp contract(off)
  return l * inv_tau;
}
__device__ __forceinline__ float add_noise(float scaled, float g) {
#pragma clang fp contract(off)
  return scaled + g;
}
__device__ __forceinline__ float gumbel_score(float scaled, uint32_t w) {
  return add_noise(scaled, dg_gumbel(dg_uniform_open01(w)));
}

// one logit into a thread's online (max, Z, A) triple and argmax; entries
// arrive in increasing vocab order, so ties keep the lower index
__device__ __forceinline__ void stat_push(Stat& t, float l, int v) {
  if (l > t.m) {
    if (t.m == -INFINITY) {
      t.Z = 1.f; t.A = 0.f;
    } else {
      const float f = __expf(t.m - l);
      t.A = f * (t.A + (t.m - l) * t.Z);
      t.Z = f * t.Z + 1.f;
    }
    t.m = l;
  } else {
    const float e = __expf(l - t.m);
    t.Z += e;
    t.A += e * (l - t.m);
  }
  if (l > t.av) { t.av = l; t.ai = v; }
}

// screened Gumbel score of one entry into the best / runner-up pair
struct Screen {
  float b1, b2, bl;   // best / runner-up screened score, best's scaled logit
  uint32_t bw;        // best's Philox word
  int bv;             // best's vocab index
};
__device__ __forceinline__ void screen_init(Screen& c) {
  c.b1 = c.b2 = -INFINITY; c.bl = 0.f; c.bw = 0u; c.bv = 0x7FFFFFFF;
}
__device__ __forceinline__ void screen_push(Screen& c, float l, float inv_tau, uint32_t w, int v) {
  const float scaled = scale_logit(l, inv_tau);
  const float sc = add_noise(scaled, gumbel_screen(dg_uniform_open01(w)));
  if (sc > c.b1) {
    c.b2 = c.b1; c.b1 = sc; c.bl = scaled; c.bw = w; c.bv = v;
  } else {
    c.b2 = fmaxf(c.b2, sc);
  }
}
// the exact score of the screened best; true when the runner-up is within
// twice the screening error, so the entries must be rescored exactly
__device__ __forceinline__ bool screen_close(const Screen& c, Stat& t) {
  if (c.bv == 0x7FFFFFFF) return false;   // no entries
  const float tol = kGumbelScreen + fmaxf(fabsf(c.b1), fabsf(c.b2)) * 2.5e-7f;
  t.gv = gumbel_score(c.bl, c.bw);
  t.gi = c.bv;
  return c.b2 >= c.b1 - 2.f * tol;
}
__device__ __forceinline__ void stat_wave_merge(Stat& t) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Stat y;
    y.m = __shfl_xor(t.m, o, 64); y.Z = __shfl_xor(t.Z, o, 64); y.A = __shfl_xor(t.A, o, 64);
    y.av = __shfl_xor(t.av, o, 64); y.ai = __shfl_xor(t.ai, o, 64);
    y.gv = __shfl_xor(t.gv, o, 64); y.gi = __shfl_xor(t.gi, o, 64);
    stat_merge(t, y);
  }
}

__global__ __launch_bounds__(256) void sample_partial_kernel(SampleArgs a) {
  if (a.flag && *a.flag) return;
  __shared__ Stat red[4][4];
  const int groups = a.T / 4;
  const int grp = blockIdx.x / a.vsplit;       // (b, position group)
  const int sl = blockIdx.x % a.vsplit;
  const int b = grp / groups, pg = grp % groups;
  if (a.stopped && a.stopped[b]) return;
  const int s = row_step(a, b);
  const float inv_tau = dg_inv_tau(a.tau_start, a.tau_end, a.max_steps, s);
  const uint64_t seed = a.seeds[b];
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int per = (a.V + a.vsplit - 1) / a.vsplit;
  const int v0 = sl * per, v1 = min(a.V, v0 + per);
  const float* l0 = a.logits + (long)(b * a.T + pg * 4) * a.ldl;

  // Per row j: softmax statistics and argmax as the logits stream by; for the
  // Gumbel maximum the screened score keeps this thread's best two, and only
  // the best one is scored exactly.  If the runner-up is within twice the
  // screening error of the best, the thread rescores all its entries of that
  // row exactly (rare), so the result is the exact maximum in every case.
  Stat st[4];
  Screen sc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    st[j] = Stat{-INFINITY, 0.f, 0.f, -INFINITY, 0x7FFFFFFF, -INFINITY, 0x7FFFFFFF};
    screen_init(sc[j]);
  }
  // entries v and v + 256 alternate between two register sets: the loads of
  // the next entry are in flight while one is processed (indices clamped to
  // the slice, so every load is issued)
  const bool stats = a.rowstat_in == nullptr;   // else the LM head has them
  const auto proc = [&](int v, const float* lv) {
    const dg_u32x4 w = dg_philox4x32_10((uint32_t)v, (uint32_t)pg, (uint32_t)s, 0u, k0, k1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (stats) stat_push(st[j], lv[j], v);
      screen_push(sc[j], lv[j], inv_tau, w.x[j], v);
    }
  };
  const int vlast = v1 - 1;
  float la[4], lb[4];
  const int vs = v0 + (int)threadIdx.x;
  if (vs < v1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) la[j] = l0[(long)j * a.ldl + vs];
  }
  for (int v = vs; v < v1; v += 512) {
#pragma unroll
    for (int j = 0; j < 4; ++j) lb[j] = l0[(long)j * a.ldl + min(v + 256, vlast)];
    proc(v, la);
#pragma unroll
    for (int j = 0; j < 4; ++j) la[j] = l0[(long)j * a.ldl + min(v + 512, vlast)];
    if (v + 256 < v1) proc(v + 256, lb);
  }
  unsigned slow = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (screen_close(sc[j], st[j])) slow |= 1u << j;
  if (slow) {
    for (int v = v0 + threadIdx.x; v < v1; v += 256) {
      const dg_u32x4 w = dg_philox4x32_10((uint32_t)v, (uint32_t)pg, (uint32_t)s, 0u, k0, k1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!((slow >> j) & 1u)) continue;
        const float sc = gumbel_score(scale_logit(l0[(long)j * a.ldl + v], inv_tau), w.x[j]);
        if (sc > st[j].gv || (sc == st[j].gv && v < st[j].gi)) { st[j].gv = sc; st[j].gi = v; }
      }
    }
  }
  // wavefront reduction
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    stat_wave_merge(st[j]);
    if (lane == 0) red[wave][j] = st[j];
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    const int j = threadIdx.x;
    Stat t = red[0][j];
    for (int w = 1; w < 4; ++w) stat_merge(t, red[w][j]);
    float* o = a.part + ((long)(b * a.T + pg * 4 + j) * a.vsplit + sl) * 8;
    o[0] = t.m; o[1] = t.Z; o[2] = t.A; o[3] = t.av;
    o[4] = __int_as_float(t.ai); o[5] = t.gv; o[6] = __int_as_float(t.gi); o[7] = 0.f;
  }
}

hipError_t sample_partial(const SampleArgs& a, hipStream_t s) {
  if (a.T % 4 != 0 || a.B > 16) return hipErrorInvalidValue;
  const int blocks = a.B * (a.T / 4) * a.vsplit;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(sample_partial_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void sample_finish_kernel(SampleArgs a) {
  if (a.flag && *a.flag) return;
  __shared__ float Hs[1024];
  __shared__ float red[16];
  __shared__ int unstable;
  const int b = blockIdx.x;
  if (a.stopped && a.stopped[b]) return;
  const int s = row_step(a, b);
  const uint64_t seed = a.seeds[b];
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int i = threadIdx.x;
  if (i == 0) unstable = 0;
  Stat t = Stat{-INFINITY, 0.f, 0.f, -INFINITY, 0x7FFFFFFF, -INFINITY, 0x7FFFFFFF};
  float H = 0.f;
  const long r = (long)b * a.T + i;
  if (i < a.T) {
    for (int sl = 0; sl < a.vsplit; ++sl) {
      const float* p = a.part + (r * a.vsplit + sl) * 8;
      Stat y{p[0], p[1], p[2], p[3], __float_as_int(p[4]), p[5], __float_as_int(p[6])};
      stat_merge(t, y);
    }
    if (a.rowstat_in) {
      const float4 rs = a.rowstat_in[r];
      H = rs.z;
      t.ai = __float_as_int(rs.w);
    } else {
      H = logf(t.Z) - t.A / t.Z;
    }
    Hs[i] = H;
  }
  __syncthreads();
  const float meanH = block_sum(i < a.T ? H : 0.f, red) / (float)a.T;
  bool lock = false;
  if (i < a.T) {
    if (a.lock_rule == 0) {
      lock = H < a.lock_thresh;
    } else {
      // sorted cumulative entropy: sum of H_j over positions ordered before or at i
      float cum = 0.f;
      for (int j = 0; j < a.T; ++j) {
        const float hj = Hs[j];
        if (hj < H || (hj == H && j <= i)) cum += hj;
      }
      lock = cum <= a.lock_thresh;
    }
    if (a.argmax[r] != t.ai) atomicOr(&unstable, 1);
  }
  __syncthreads();
  bool stop;
  if (a.stop_rule == 0) stop = meanH < a.stop_thresh;
  else stop = (meanH < a.stop_thresh) && (s > 0) && (unstable == 0);
  stop = stop || (s + 1 >= a.max_steps);
  if (i < a.T) {
    int tok;
    if (stop || lock) {
      tok = t.gi;
    } else {
      const dg_u32x4 w = dg_philox4x32_10((uint32_t)i, 0u, (uint32_t)s, 1u, k0, k1);
      tok = (int)dg_uniform_index(w.x[0], (uint32_t)a.V);
    }
    a.tokens[r] = tok;
    a.xhat[r] = t.gi;
    a.argmax[r] = t.ai;
    a.entropy[r] = H;
    a.locked[r] = lock ? 1 : 0;
    if (a.rowstat) a.rowstat[r] = make_float4(t.m, t.Z, H, __int_as_float(t.ai));
  }
  if (i == 0) {
    a.stopped[b] = stop ? 1 : 0;
    a.steps[b] = s + 1;
  }
}

__global__ void all_stopped_kernel(const int32_t* stopped, int B, int32_t* flag) {
  if (threadIdx.x == 0) {
    int all = 1;
    for (int b = 0; b < B; ++b) all &= (stopped[b] != 0);
    *flag = all;
  }
}

hipError_t sample_finish(const SampleArgs& a, hipStream_t s) {
  if (a.T > 1024 || a.B > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_finish_kernel, dim3(a.B), dim3(a.T <= 256 ? 256 : 1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.all_stopped) return e;
  hipLaunchKernelGGL(all_stopped_kernel, dim3(1), dim3(64), 0, s, a.stopped, a.B, a.all_stopped);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Next-token sampler of the autoregressive step (one position per row; the
// step the article's section 5 compares a denoising step with): Gumbel-max
// over softmax(l / tau), plus the argmax and entropy of the logits.  The
// noise of vocab entry v at decode position p is word v & 3 of Philox block
// (v >> 2, p, 0, 2) keyed by the row seed, so one 10-round call covers four
// consecutive entries, read as one float4.  One workgroup per (row, vocab
// slice of whole blocks of four); the finish kernel merges the slices.
__global__ __launch_bounds__(256) void ar_sample_partial_kernel(ArSampleArgs a) {
  __shared__ Stat red[4];
  const int b = blockIdx.x / a.vsplit, sl = blockIdx.x % a.vsplit;
  const uint64_t seed = a.seeds[b];
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int ng = a.V / 4;
  const int per = (ng + a.vsplit - 1) / a.vsplit;
  const int g0 = sl * per, g1 = min(ng, g0 + per);
  const float* l = a.logits + (long)b * a.ldl;
  const int pos = a.pos_dev ? *a.pos_dev : a.pos;
  Stat t = Stat{-INFINITY, 0.f, 0.f, -INFINITY, 0x7FFFFFFF, -INFINITY, 0x7FFFFFFF};
  Screen c;
  screen_init(c);
  for (int g = g0 + (int)threadIdx.x; g < g1; g += 256) {
    const float4 x = *reinterpret_cast<const float4*>(l + 4L * g);
    const dg_u32x4 w = dg_philox4x32_10((uint32_t)g, (uint32_t)pos, 0u, 2u, k0, k1);
    const float lv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      stat_push(t, lv[j], 4 * g + j);
      screen_push(c, lv[j], a.inv_tau, w.x[j], 4 * g + j);
    }
  }
  if (screen_close(c, t)) {
    for (int g = g0 + (int)threadIdx.x; g < g1; g += 256) {
      const dg_u32x4 w = dg_philox4x32_10((uint32_t)g, (uint32_t)pos, 0u, 2u, k0, k1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = 4 * g + j;
        const float sc = gumbel_score(scale_logit(l[v], a.inv_tau), w.x[j]);
        if (sc > t.gv || (sc == t.gv && v < t.gi)) { t.gv = sc; t.gi = v; }
      }
    }
  }
  stat_wave_merge(t);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    Stat r = red[0];
    for (int w = 1; w < 4; ++w) stat_merge(r, red[w]);
    float* o = a.part + ((long)b * a.vsplit + sl) * 8;
    o[0] = r.m; o[1] = r.Z; o[2] = r.A; o[3] = r.av;
    o[4] = __int_as_float(r.ai); o[5] = r.gv; o[6] = __int_as_float(r.gi); o[7] = 0.f;
  }
}

__global__ __launch_bounds__(64) void ar_sample_finish_kernel(ArSampleArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  Stat t = Stat{-INFINITY, 0.f, 0.f, -INFINITY, 0x7FFFFFFF, -INFINITY, 0x7FFFFFFF};
  for (int sl = lane; sl < a.vsplit; sl += 64) {
    const float* p = a.part + ((long)b * a.vsplit + sl) * 8;
    Stat y{p[0], p[1], p[2], p[3], __float_as_int(p[4]), p[5], __float_as_int(p[6])};
    stat_merge(t, y);
  }
  stat_wave_merge(t);
  if (lane == 0) {
    a.next[b] = t.gi;
    if (a.argmax) a.argmax[b] = t.ai;
    if (a.entropy) a.entropy[b] = logf(t.Z) - t.A / t.Z;
  }
}

hipError_t ar_sample(const ArSampleArgs& a, hipStream_t s) {
  if (a.B < 1 || a.B > 16 || a.V % 4 != 0 || a.ldl % 4 != 0 || a.vsplit < 1 || !a.next || !a.part)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(ar_sample_partial_kernel, dim3(a.B * a.vsplit), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ar_sample_finish_kernel, dim3(a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Softmax statistics per vocabulary slice and the soft-prediction embedding.
// The slices are those of the soft-prediction product's split contraction, so
// each slice's probabilities can be scaled by its own maximum: the product
// sums e^(l_v - m_s) E_v over the slice, and the finishing pass weighs slice
// s by e^(m_s - M) / Z (the online-softmax merge of the slices' statistics).

// (max, argmax) of the 64 lanes of a wave, in every lane; ties to the lower index
__device__ __forceinline__ void wave_argmax(float& mx, int& ix) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float om = __shfl_xor(mx, o, 64);
    const int oi = __shfl_xor(ix, o, 64);
    const bool take = (om > mx) | ((om == mx) & (oi < ix));
    mx = take ? om : mx;
    ix = take ? oi : ix;
  }
}

// A thread's entries of its slice (float4 entries 4 tid + 1024 j) are loaded in
// one batch and kept in registers for both passes when the slice holds at most
// kSliceRegs of them per thread (REG); otherwise each pass streams them.
constexpr int kSliceRegs = 16;
template <bool REG>
__global__ __launch_bounds__(256) void softmax_slice_kernel(const float* logits, long ldl, int V, int kchunk,
                                                            int nslices, int T, const int32_t* stopped, bf16_t* P,
                                                            float4* sstat, const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ float smx[4], sz[4], sa[4];
  __shared__ int six[4];
  const int r = blockIdx.x / nslices, sl = blockIdx.x % nslices;
  if (stopped && stopped[r / T]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v0 = sl * kchunk, v1 = min(V, v0 + kchunk);   // multiples of 4
  const float* l = logits + (long)r * ldl;
  constexpr int NR = REG ? kSliceRegs : 1;
  float4 xr[NR];
  if (REG) {
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int v = v0 + 4 * tid + 1024 * j;
      if (v < v1) xr[j] = *reinterpret_cast<const float4*>(l + v);
    }
  }
  // the slice's maximum and argmax (entries in increasing order per thread)
  float mx = -INFINITY;
  int ix = 0x7FFFFFFF;
  auto scan = [&](const float4 x, int v) {
    if (x.x > mx) { mx = x.x; ix = v; }
    if (x.y > mx) { mx = x.y; ix = v + 1; }
    if (x.z > mx) { mx = x.z; ix = v + 2; }
    if (x.w > mx) { mx = x.w; ix = v + 3; }
  };
  if (REG) {
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int v = v0 + 4 * tid + 1024 * j;
      if (v < v1) scan(xr[j], v);
    }
  } else {
    for (int v = v0 + 4 * tid; v < v1; v += 1024) scan(*reinterpret_cast<const float4*>(l + v), v);
  }
  wave_argmax(mx, ix);
  if (lane == 0) { smx[wave] = mx; six[wave] = ix; }
  __syncthreads();
  float M = smx[0];
  int I = six[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const bool take = (smx[w] > M) | ((smx[w] == M) & (six[w] < I));
    M = take ? smx[w] : M;
    I = take ? six[w] : I;
  }
  // e^(l - M) summed, with its (l - M)-weighted sum (entropy), stored scaled
  float z = 0.f, a = 0.f;
  bf16_t* prow = P ? P + (long)r * V : nullptr;
  auto accumulate = [&](const float4 x, int v) {
    const float d0 = x.x - M, d1 = x.y - M, d2 = x.z - M, d3 = x.w - M;
    const float e0 = __expf(d0), e1 = __expf(d1), e2 = __expf(d2), e3 = __expf(d3);
    z += (e0 + e1) + (e2 + e3);
    a += (e0 * d0 + e1 * d1) + (e2 * d2 + e3 * d3);
    if (prow) {
      uint2 o;
      o.x = (uint32_t)f2bf(e0) | ((uint32_t)f2bf(e1) << 16);
      o.y = (uint32_t)f2bf(e2) | ((uint32_t)f2bf(e3) << 16);
      *reinterpret_cast<uint2*>(prow + v) = o;
    }
  };
  if (REG) {
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int v = v0 + 4 * tid + 1024 * j;
      if (v < v1) accumulate(xr[j], v);
    }
  } else {
    for (int v = v0 + 4 * tid; v < v1; v += 1024) accumulate(*reinterpret_cast<const float4*>(l + v), v);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    z += __shfl_xor(z, o, 64);
    a += __shfl_xor(a, o, 64);
  }
  if (lane == 0) { sz[wave] = z; sa[wave] = a; }
  __syncthreads();
  if (tid == 0)
    sstat[(long)r * nslices + sl] = make_float4(M, (sz[0] + sz[1]) + (sz[2] + sz[3]), (sa[0] + sa[1]) + (sa[2] + sa[3]),
                                                __int_as_float(I));
}

hipError_t softmax_slices(const float* logits, long ldl, int rows, int V, int kchunk, int nslices, int T,
                          const int32_t* stopped, bf16_t* P, float4* sstat, const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (V % 4 || kchunk % 4 || ldl % 4 || nslices < 1 || (long)kchunk * nslices < V || T < 1)
    return hipErrorInvalidValue;
  if (kchunk <= 1024 * kSliceRegs)
    hipLaunchKernelGGL(softmax_slice_kernel<true>, dim3((unsigned)(rows * nslices)), dim3(256), 0, s, logits, ldl, V,
                       kchunk, nslices, T, stopped, P, sstat, flag);
  else
    hipLaunchKernelGGL(softmax_slice_kernel<false>, dim3((unsigned)(rows * nslices)), dim3(256), 0, s, logits, ldl,
                       V, kchunk, nslices, T, stopped, P, sstat, flag);
  return hipGetLastError();
}

// Workgroup (r, y): wave 0 merges the row's slice statistics (lane s holds
// slice s; a butterfly of the online-softmax merge), the weights
// e^(m_s - M) / Z go to LDS, and every thread sums 4 columns of s_next over
// the slices.  Workgroup (r, 0) also writes the row's statistics.
__global__ __launch_bounds__(256) void softmax_finish_kernel(const float4* sstat, int nslices, int rows, int T,
                                                             const int32_t* stopped, const float* part, int d,
                                                             bf16_t* out, float4* rowstat, const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ float w[64];
  const int r = blockIdx.x;
  if (stopped && stopped[r / T]) return;
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const float4 mine = s < nslices ? sstat[(long)r * nslices + s]
                                    : make_float4(-INFINITY, 0.f, 0.f, __int_as_float(0x7FFFFFFF));
    float4 t = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      float4 y;
      y.x = __shfl_xor(t.x, o, 64); y.y = __shfl_xor(t.y, o, 64); y.z = __shfl_xor(t.z, o, 64);
      y.w = __shfl_xor(t.w, o, 64);
      t = softmax_stats_merge(t, y);
    }
    if (s < nslices) w[s] = __expf(mine.x - t.x) / t.y;
    if (s == 0 && blockIdx.y == 0) rowstat[r] = make_float4(t.x, t.y, logf(t.y) - t.z / t.y, t.w);
  }
  if (!out) return;
  __syncthreads();
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= d) return;
  const long n = (long)rows * d;
  const float* pp = part + (long)r * d + c;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nslices; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(pp + s * n);
    const float ws = w[s];
    acc.x += ws * v.x; acc.y += ws * v.y; acc.z += ws * v.z; acc.w += ws * v.w;
  }
  uint2 o;
  o.x = (uint32_t)f2bf(acc.x) | ((uint32_t)f2bf(acc.y) << 16);
  o.y = (uint32_t)f2bf(acc.z) | ((uint32_t)f2bf(acc.w) << 16);
  *reinterpret_cast<uint2*>(out + (long)r * d + c) = o;
}

hipError_t softmax_finish(const float4* sstat, int nslices, int rows, int T, const int32_t* stopped,
                          const float* part, int d, bf16_t* out, float4* rowstat, const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (nslices < 1 || nslices > 64 || T < 1 || d % 4) return hipErrorInvalidValue;
  const dim3 grid(rows, out ? (d / 4 + 255) / 256 : 1);
  hipLaunchKernelGGL(softmax_finish_kernel, grid, dim3(256), 0, s, sstat, nslices, rows, T, stopped, part, d, out,
                     rowstat, flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
struct Seeds16 { uint64_t s[16]; };

__global__ void init_canvas_kernel(int32_t* tokens, int B, int T, int V, Seeds16 sd) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * T) return;
  const int b = idx / T, i = idx % T;
  const uint64_t seed = sd.s[b];
  const dg_u32x4 w = dg_philox4x32_10((uint32_t)i, 0u, 0xFFFFFFFFu, 1u, (uint32_t)seed, (uint32_t)(seed >> 32));
  tokens[idx] = (int32_t)dg_uniform_index(w.x[0], (uint32_t)V);
}

hipError_t init_canvas(int32_t* tokens, int B, int T, int V, const uint64_t* seeds, hipStream_t s) {
  if (B > 16) return hipErrorInvalidValue;
  Seeds16 sd{};
  for (int b = 0; b < B; ++b) sd.s[b] = seeds[b];
  hipLaunchKernelGGL(init_canvas_kernel, dim3((B * T + 255) / 256), dim3(256), 0, s, tokens, B, T, V, sd);
  return hipGetLastError();
}

__global__ void set_step_kernel(int32_t* steps, const int32_t* stopped, int B, int step) {
  if ((int)threadIdx.x < B && !stopped[threadIdx.x]) steps[threadIdx.x] = step;
}

hipError_t set_step(int32_t* steps, const int32_t* stopped, int B, int step, hipStream_t s) {
  if (B > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(set_step_kernel, dim3(1), dim3(64), 0, s, steps, stopped, B, step);
  return hipGetLastError();
}

}  // namespace dg
