// Row-wise kernels of one transformer layer of the denoising step (gfx950):
// embedding gather, RMSNorm, per-head QK RMSNorm + rotary embedding with the
// scatter of K and V^T into the attention caches, split-attention merge, MoE
// router top-k, expert permutation (wavefront ballot scans) and the combine
// that also produces the next RMSNorm.  All are bandwidth-trivial next to the
// weight streams; they are written to keep the number of passes over the
// activations low (one workgroup per token row, values kept in registers).
#include <math.h>

#include "dg_kernels.hpp"

namespace dg {

#define DG_MAXD_PER_THREAD 16  // d_model <= 4096 with 256 threads

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* tok, const bf16_t* E, int d, float* h,
                                                    const int32_t* flag) {
  if (flag && *flag) return;
  const int r = blockIdx.x;
  const bf16_t* e = E + (long)tok[r] * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) h[(long)r * d + c] = bf2f(e[c]);
}

hipError_t embed_rows(const int32_t* tokens, const bf16_t* E, int rows, int d, float* h, const int32_t* flag,
                      hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, s, tokens, E, d, h, flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rmsnorm_kernel(float* h, const bf16_t* w, int rows, int d, float eps,
                                                      bf16_t* out, bf16_t* split, float* dump, Partials part,
                                                      const bf16_t* pgate, const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ float red[16];
  const int r = blockIdx.x;
  float* x = h + (long)r * d;
  float v[DG_MAXD_PER_THREAD];
  float ss = 0.f;
  int n = 0;
  for (int c = threadIdx.x; c < d; c += 256, ++n) {
    float xv = x[c];
    if (part.n > 0) {
      float acc = 0.f;
      for (int s = 0; s < part.n; ++s) acc += part.p[s * part.stride + (long)r * d + c];
      xv += pgate ? sigmoidf_(bf2f(pgate[c])) * acc : acc;
      x[c] = xv;
    }
    v[n] = xv;
    ss += xv * xv;
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  n = 0;
  for (int c = threadIdx.x; c < d; c += 256, ++n) {
    const float y = v[n] * inv * bf2f(w[c]);
    const uint16_t hi = f2bf(y);
    out[(long)r * d + c] = hi;
    if (split) {
      split[(long)r * d + c] = hi;
      split[(long)(rows + r) * d + c] = f2bf(y - bf2f(hi));
    }
    if (dump) dump[(long)r * d + c] = v[n];
  }
}

hipError_t rmsnorm_rows(float* h, const bf16_t* w, int rows, int d, float eps, bf16_t* out, bf16_t* split_hi_lo,
                        float* dump, Partials part, const bf16_t* part_gate, const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d > 256 * DG_MAXD_PER_THREAD) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, h, w, rows, d, eps, out, split_hi_lo, dump, part,
                     part_gate, flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One workgroup per token row.  Waves take heads round-robin: q heads, then k
// heads (both RMSNorm over head_dim + rotate-half RoPE), then v heads (copy).
// Lane l holds elements l + 64 j of a head; the rotary partner of element e is
// e +- hd/2, i.e. slot j +- hd/128 of the same lane when hd >= 128, or lane
// l ^ (hd/2) when hd == 64.
template <int HD>
__global__ __launch_bounds__(256) void qk_rope_kernel(QkRopeArgs a) {
  if (a.flag && *a.flag) return;
  constexpr int HALF = HD / 2;
  constexpr int NS = (HD + 63) / 64;
  __shared__ float cs[HALF], sn[HALF];
  const int r = blockIdx.x;
  const int tloc = r % a.per_batch, bidx = r / a.per_batch;
  const double pos = (double)(a.pos0 + tloc);
  for (int j = threadIdx.x; j < HALF; j += blockDim.x) {
    const double freq = exp(-(2.0 * (double)j / (double)HD) * log((double)a.theta));
    double sv, cv;
    sincos(pos * freq, &sv, &cv);
    cs[j] = (float)cv;
    sn[j] = (float)sv;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qkvd = (a.H + 2 * a.Hkv) * HD;
  const bf16_t* src = a.qkv + (long)r * qkvd;
  const int nh = a.H + 2 * a.Hkv;
  for (int hh = wave; hh < nh; hh += 4) {
    const bf16_t* xs = src + hh * HD;
    if (hh >= a.H + a.Hkv) {  // value head: scatter into V^T
      const int g = hh - a.H - a.Hkv;
      bf16_t* vt = a.vtdst + bidx * a.v_bstride + g * a.v_hstride + (a.t_offset + tloc);
      for (int e = lane; e < HD; e += 64) vt[(long)e * a.v_pitch] = xs[e];
      continue;
    }
    const bool isq = hh < a.H;
    const bf16_t* nw = isq ? a.qnorm : a.knorm;
    float x[NS];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int e = lane + 64 * j;
      x[j] = (e < HD) ? bf2f(xs[e]) : 0.f;
      ss += x[j] * x[j];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int e = lane + 64 * j;
      x[j] = (e < HD) ? x[j] * inv * bf2f(nw[e]) : 0.f;
    }
    float y[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int e = lane + 64 * j;
      float partner;
      if (HD >= 128) {
        partner = x[(j + HALF / 64) % NS];
      } else {
        partner = __shfl_xor(x[j], HALF, 64);
      }
      if (e < HALF) {
        y[j] = x[j] * cs[e] - partner * sn[e];
      } else {
        const int jj = e - HALF;
        y[j] = x[j] * cs[jj < HALF ? jj : 0] + partner * sn[jj < HALF ? jj : 0];
      }
    }
    if (isq) {
      bf16_t* qd = a.q + ((long)r * a.H + hh) * HD;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int e = lane + 64 * j;
        if (e < HD) qd[e] = f2bf(y[j]);
      }
    } else {
      const int g = hh - a.H;
      bf16_t* kd = a.kdst + bidx * a.k_bstride + g * a.k_hstride + (long)(a.t_offset + tloc) * HD;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int e = lane + 64 * j;
        if (e < HD) kd[e] = f2bf(y[j]);
      }
    }
  }
}

hipError_t qk_norm_rope(const QkRopeArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  switch (a.hd) {
    case 64: hipLaunchKernelGGL(qk_rope_kernel<64>, dim3(a.rows), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(qk_rope_kernel<128>, dim3(a.rows), dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(qk_rope_kernel<256>, dim3(a.rows), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge of key-split attention partials (scores kept in log2 units): per row,
// the split weights 2^(m_s - M) / L of every head are formed once in LDS, then
// the outputs are summed with coalesced reads of the partials.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* op, const float* ml, int splits, int rows,
                                                         int H, int hd, bf16_t* out, const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ float wts[1024];
  const int r = blockIdx.x;
  const long srow = (long)rows * H;
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    const long base = (long)r * H + h;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[(s * srow + base) * 2]);
    float L = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float m = ml[(s * srow + base) * 2];
      const float w = (m == -INFINITY) ? 0.f : exp2f(m - M);
      wts[h * splits + s] = w;
      L += w * ml[(s * srow + base) * 2 + 1];
    }
    const float il = L > 0.f ? 1.0f / L : 0.f;
    for (int s = 0; s < splits; ++s) wts[h * splits + s] *= il;
  }
  __syncthreads();
  const long rowoff = (long)r * H * hd;
  const long sstride = srow * hd;
  for (int idx = threadIdx.x; idx < H * hd; idx += blockDim.x) {
    const int h = idx / hd;
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) acc += wts[h * splits + s] * op[s * sstride + rowoff + idx];
    out[rowoff + idx] = f2bf(acc);
  }
}

hipError_t attention_merge(const float* opart, const float* mlpart, int splits, int rows, int H, int hd,
                           bf16_t* out, const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (H * splits > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(rows), dim3(256), 0, s, opart, mlpart, splits, rows, H, hd, out, flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router: logits = hi-part + lo-part products (an fp32-accurate product from two
// bf16 MFMA passes), top-k by repeated wavefront argmax (ties -> lower expert),
// gates = softmax over the k selected logits.  One wave per token row.
__global__ __launch_bounds__(256) void topk_kernel(Partials rl, int rows, int E, int k, int32_t* idx,
                                                   float* gate, int32_t* idx_dump, float* gate_dump,
                                                   const int32_t* flag) {
  if (flag && *flag) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    float hi = 0.f, lo = 0.f;
    if (e < E) {
      for (int s = 0; s < rl.n; ++s) {
        hi += rl.p[s * rl.stride + (long)r * E + e];
        lo += rl.p[s * rl.stride + (long)(rows + r) * E + e];
      }
    }
    v[j] = (e < E) ? hi + lo : -INFINITY;
  }
  float selv[16];
  int seli[16];
  for (int t = 0; t < k; ++t) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E && (v[j] > bv || (v[j] == bv && e < bi))) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    selv[t] = bv;
    seli[t] = bi;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == bi) v[j] = -INFINITY;
  }
  if (lane == 0) {
    float s = 0.f, ex[16];
    for (int t = 0; t < k; ++t) {
      ex[t] = expf(selv[t] - selv[0]);
      s += ex[t];
    }
    for (int t = 0; t < k; ++t) {
      const float gt = ex[t] / s;
      idx[(long)r * k + t] = seli[t];
      gate[(long)r * k + t] = gt;
      if (idx_dump) idx_dump[(long)r * k + t] = seli[t];
      if (gate_dump) gate_dump[(long)r * k + t] = gt;
    }
  }
}

hipError_t router_topk(Partials rlog, int rows, int E, int k, int32_t* idx, float* gate, int32_t* idx_dump,
                       float* gate_dump, const int32_t* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (E > 256 || k > 16 || k > E) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, rlog, rows, E, k, idx, gate, idx_dump,
                     gate_dump, flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Expert permutation in one workgroup of 1024 threads (16 waves).
// Assignment a = row * k + j goes to slot offsets[e] + (number of earlier
// assignments to the same expert e), so every expert's rows stay in token
// order (deterministic).  Within a wave, lanes with equal experts are found
// with 8 ballots (one per bit of e); per-wave counts are scanned across the
// 16 waves of a tile and across tiles.
__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* idx, int na, int k, int E, int32_t* counts,
                                                       int32_t* offsets, int32_t* slot_of, int32_t* slot_row,
                                                       int4* items, int32_t* n_items, int chunk,
                                                       const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ int wcnt[16][256];
  __shared__ int cnt[256];
  __shared__ int off[257];
  __shared__ int ibase[257];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < 256; e += 1024) cnt[e] = 0;
  for (int base = 0; base < na; base += 1024) {
    for (int i = tid; i < 16 * 256; i += 1024) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const int a = base + tid;
    const bool valid = a < na;
    const int e = valid ? idx[a] : 255;
    unsigned long long mask = __ballot(valid);
    if (!valid) mask = ~mask;
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (e >> bit) & 1;
      const unsigned long long bb = __ballot(on);
      mask &= on ? bb : ~bb;
    }
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    if (valid && rank == 0) wcnt[wave][e] = __popcll(mask);
    __syncthreads();
    if (tid < E) {
      int run = cnt[tid];
      for (int w = 0; w < 16; ++w) {
        const int c = wcnt[w][tid];
        wcnt[w][tid] = run;
        run += c;
      }
      cnt[tid] = run;
    }
    __syncthreads();
    if (valid) slot_of[a] = wcnt[wave][e] + rank;
    __syncthreads();
  }
  if (tid == 0) {
    int run = 0, ni = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = run;
      ibase[e] = ni;
      run += cnt[e];
      ni += (cnt[e] + chunk - 1) / chunk;
    }
    off[E] = run;
    ibase[E] = ni;
    *n_items = ni;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) {
    offsets[e] = off[e];
    if (e < E) {
      counts[e] = cnt[e];
      int i = ibase[e];
      for (int r = 0; r < cnt[e]; r += chunk, ++i) items[i] = make_int4(e, off[e] + r, min(chunk, cnt[e] - r), 0);
    }
  }
  for (int a = tid; a < na; a += 1024) {
    const int e = idx[a];
    const int slot = off[e] + slot_of[a];
    slot_of[a] = slot;
    slot_row[slot] = a / k;
  }
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
__global__ __launch_bounds__(256) void combine_kernel(float* h, Partials ys, const float* Y,
                                                      const int32_t* slot_of, const float* gate, int d, int k,
                                                      const bf16_t* nw, float eps, bf16_t* xn, float* dump,
                                                      const int32_t* flag) {
  if (flag && *flag) return;
  __shared__ float red[16];
  __shared__ int slots[16];
  __shared__ float gts[16];
  const int r = blockIdx.x;
  if (threadIdx.x < k) {
    slots[threadIdx.x] = slot_of[(long)r * k + threadIdx.x];
    gts[threadIdx.x] = gate[(long)r * k + threadIdx.x];
  }
  __syncthreads();
  float v[DG_MAXD_PER_THREAD];
  float ss = 0.f;
  int n = 0;
  for (int c = threadIdx.x; c < d; c += 256, ++n) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc += gts[j] * Y[(long)slots[j] * d + c];
    for (int s = 0; s < ys.n; ++s) acc += ys.p[s * ys.stride + (long)r * d + c];
    const float x = h[(long)r * d + c] + acc;
    h[(long)r * d + c] = x;
    v[n] = x;
    ss += x * x;
  }
  if (!nw && !dump) return;
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  n = 0;
  for (int c = threadIdx.x; c < d; c += 256, ++n) {
    if (nw) xn[(long)r * d + c] = f2bf(v[n] * inv * bf2f(nw[c]));
    if (dump) dump[(long)r * d + c] = v[n];
  }
}

hipError_t moe_combine(float* h, Partials ys, const float* Y, const int32_t* slot_of, const float* gate, int rows,
                       int d, int k, const bf16_t* next_w, float eps, bf16_t* xn, float* dump, const int32_t* flag,
                       hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d > 256 * DG_MAXD_PER_THREAD || k > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(rows), dim3(256), 0, s, h, ys, Y, slot_of, gate, d, k, next_w, eps, xn,
                     dump, flag);
  return hipGetLastError();
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

__global__ void transpose_kernel(const bf16_t* in, bf16_t* out, long rows, long cols) {
  __shared__ bf16_t tile[32][33];
  const long c0 = (long)blockIdx.x * 32, r0 = (long)blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int j = ty; j < 32; j += 8) {
    const long r = r0 + j, c = c0 + tx;
    if (r < rows && c < cols) tile[j][tx] = in[r * cols + c];
  }
  __syncthreads();
  for (int j = ty; j < 32; j += 8) {
    const long c = c0 + j, r = r0 + tx;
    if (r < rows && c < cols) out[c * rows + r] = tile[tx][j];
  }
}

hipError_t transpose_bf16(const bf16_t* in, bf16_t* out, long rows, long cols, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, in, out, rows, cols);
  return hipGetLastError();
}

}  // namespace dg
