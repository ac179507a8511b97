// Shared device helpers for the gfx950 (CDNA4) kernels of libdg.
//
// bf16 values travel as raw uint16_t bit patterns; arithmetic is fp32.
// MFMA: v_mfma_f32_16x16x32_bf16.  Operand convention used everywhere:
//   A (16 x 32): lane l holds row (l % 16), k-slots 8*(l/16) .. +7
//   B (32 x 16): lane l holds col (l % 16), k-slots 8*(l/16) .. +7
//   D (16 x 16): lane l holds rows 4*(l/16) + i (i = 0..3), col (l % 16)
// Only the pairing of A's and B's k-slots matters for the contraction, so a
// kernel may map any 32 contraction indices onto the slots as long as A and
// B use the same map.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16_t;

#define DG_WAVE 64

// Workgroups are dealt to the 8 XCDs in turn (block b runs on XCD b mod 8).
// The grid is padded to a multiple of 8 and renumbered so that every XCD works
// through one contiguous range of logical tiles: workgroups that read the same
// operand tiles then run side by side on one XCD and share its L2.
__device__ inline long xcd_logical_block(long total) {
  const long b = blockIdx.x;
  const long per = gridDim.x >> 3;
  const long l = (b & 7) * per + (b >> 3);
  return l < total ? l : -1;
}
static inline unsigned xcd_grid(long total) { return (unsigned)((total + 7) & ~7L); }

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, DG_WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, DG_WAVE));
  return v;
}

// block-wide sum for blockDim.x a multiple of 64 (<= 1024); deterministic order.
__device__ __forceinline__ float block_sum(float v, float* red /* >= 16 floats */) {
  v = wave_sum(v);
  const int w = threadIdx.x / DG_WAVE, l = threadIdx.x % DG_WAVE;
  const int nw = blockDim.x / DG_WAVE;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ float gelu_tanh(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  float u = k0 * (x + 0.044715f * x * x * x);
  // tanh(u) = 1 - 2 / (exp(2u) + 1), saturating correctly at both ends
  float t = 1.0f - 2.0f / (__expf(2.0f * u) + 1.0f);
  return 0.5f * x * (1.0f + t);
}

// Online-softmax merge of two partial statistics {max m, Z = sum e^(l - m),
// A = sum e^(l - m)(l - m), argmax (int bits)} over disjoint sets of logits:
// both sums are rescaled to the larger maximum M (A also gains (m - M) Z from
// the shift); the argmax keeps the larger logit, ties to the lower index.  An
// empty partial has m = -inf.
__device__ __forceinline__ float4 softmax_stats_merge(float4 x, float4 y) {
  if (y.x == -INFINITY) return x;
  if (x.x == -INFINITY) return y;
  const float M = fmaxf(x.x, y.x);
  const float fx = __expf(x.x - M), fy = __expf(y.x - M);
  float4 r;
  r.x = M;
  r.y = fx * x.y + fy * y.y;
  r.z = fx * (x.z + (x.x - M) * x.y) + fy * (y.z + (y.x - M) * y.y);
  const int xi = __float_as_int(x.w), yi = __float_as_int(y.w);
  r.w = (y.x > x.x || (y.x == x.x && yi < xi)) ? y.w : x.w;
  return r;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }
