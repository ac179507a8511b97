// Weight-streaming bf16 GEMM on MFMA (v_mfma_f32_16x16x32_bf16) for gfx950.
//
// Every product of the denoising step pairs few activation rows (256 canvas
// tokens; ~16-100 per expert) with a large weight matrix, so the kernel is built
// to keep many weight bytes in flight and to read each byte once:
//   * a workgroup owns one output tile: <= 64 rows (one "item" = a chunk of one
//     expert's rows, or of the dense rows) x 16*NF columns (GEGLU: NF gate and NF
//     up fragments);
//   * its 4 waves split the contraction dimension in four contiguous ranges, so
//     every A and B byte of the tile is loaded by exactly one wave, straight from
//     global memory into MFMA operand registers with 16-byte loads; two k-steps
//     of 32 are in flight while the previous two are multiplied (loads are
//     branch-free so the wait before each MFMA group covers only its buffer);
//   * the four partial tiles are summed through LDS and the epilogue (store,
//     residual add, gated add, GELU-tanh gating) is split over the waves;
//   * expert rows are gathered through a row map (no copies), and large experts
//     are cut into several items that run on different workgroups.
#include "dg_kernels.hpp"

namespace dg {

template <int EPI, int MF, int NF>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g) {
  constexpr int NFT = (EPI == EPI_GEGLU_BF16) ? 2 * NF : NF;
  __shared__ floatx4 red[4][MF * NFT][64];
  if (g.flag && *g.flag) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntiles = (g.N + 16 * NF - 1) / (16 * NF);
  const long b = blockIdx.x;
  const int item = (int)(b % g.items_max);
  const long rest = b / g.items_max;
  const int tile = (int)(rest % ntiles);
  const int zk = (int)(rest / ntiles);

  int grp, r0, nrows;
  if (g.items) {
    if (item >= *g.n_items) return;
    const int4 it = g.items[item];
    grp = it.x;
    r0 = it.y;
    nrows = it.z;
  } else {
    grp = 0;
    r0 = item * 16 * MF;
    nrows = min(16 * MF, g.M - r0);
  }
  if (nrows <= 0) return;
  const int nmf = (nrows + 15) >> 4;
  const int n_base = tile * 16 * NF;

  // contraction range of this workgroup and of this wave, in 32-wide k-steps
  const int kb = zk * g.k_chunk;
  const int ke = min(g.K, kb + g.k_chunk);
  const int nks = (ke - kb) >> 5;
  const int ks0 = (kb >> 5) + (nks * wave) / 4;
  const int ks1 = (kb >> 5) + (nks * (wave + 1)) / 4;

  const int lr = lane & 15, lg = lane >> 4;
  const bf16_t* bp[NFT];
#pragma unroll
  for (int f = 0; f < NFT; ++f) {
    const bool up = (EPI == EPI_GEGLU_BF16) && f >= NF;
    const int n = min(n_base + (up ? f - NF : f) * 16 + lr, g.N - 1);
    const bf16_t* Wb = up ? g.W2 : g.W;
    bp[f] = Wb + (long)grp * g.w_gstride + (long)n * g.ldw + lg * 8;
  }
  const bf16_t* ap[MF];
#pragma unroll
  for (int m = 0; m < MF; ++m) {
    const int r = r0 + min(m * 16 + lr, nrows - 1);
    const int ar = g.a_rows ? g.a_rows[r] : r;
    ap[m] = g.A + (long)ar * g.lda + lg * 8;
  }

  floatx4 acc[MF][NFT];
#pragma unroll
  for (int m = 0; m < MF; ++m)
#pragma unroll
    for (int f = 0; f < NFT; ++f) acc[m][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Ping-pong register buffers X (k-steps ks, ks+1) and Y (ks+2, ks+3).  Loads
  // are branch-free (indices clamped into this wave's range, every row
  // fragment loaded) so the compiler can wait for exactly the older buffer
  // while the newer one is still in flight.
  bf16x8 xa0[MF], xa1[MF], xb0[NFT], xb1[NFT];
  bf16x8 ya0[MF], ya1[MF], yb0[NFT], yb1[NFT];
#define DG_LOAD_STEP(KS, AR, BR)                                                         \
  do {                                                                                   \
    const int k_ = min((KS), ks1 - 1) << 5;                                              \
    _Pragma("unroll") for (int f = 0; f < NFT; ++f) BR[f] = load_bf16x8(bp[f] + k_);     \
    _Pragma("unroll") for (int m = 0; m < MF; ++m) AR[m] = load_bf16x8(ap[m] + k_);      \
  } while (0)
#define DG_MMA_STEP(AR, BR)                                                              \
  do {                                                                                   \
    _Pragma("unroll") for (int m = 0; m < MF; ++m) if (m < nmf)                         \
      _Pragma("unroll") for (int f = 0; f < NFT; ++f) acc[m][f] = mfma16x16x32(AR[m], BR[f], acc[m][f]); \
  } while (0)

  if (ks0 < ks1) {
    DG_LOAD_STEP(ks0, xa0, xb0);
    DG_LOAD_STEP(ks0 + 1, xa1, xb1);
    for (int ks = ks0; ks < ks1; ks += 4) {
      DG_LOAD_STEP(ks + 2, ya0, yb0);
      DG_LOAD_STEP(ks + 3, ya1, yb1);
      DG_MMA_STEP(xa0, xb0);
      if (ks + 1 < ks1) DG_MMA_STEP(xa1, xb1);
      DG_LOAD_STEP(ks + 4, xa0, xb0);
      DG_LOAD_STEP(ks + 5, xa1, xb1);
      if (ks + 2 < ks1) DG_MMA_STEP(ya0, yb0);
      if (ks + 3 < ks1) DG_MMA_STEP(ya1, yb1);
    }
  }
#undef DG_LOAD_STEP
#undef DG_MMA_STEP

  // sum the four k-range partials
#pragma unroll
  for (int m = 0; m < MF; ++m)
#pragma unroll
    for (int f = 0; f < NFT; ++f) red[wave][m * NFT + f][lane] = acc[m][f];
  __syncthreads();
  for (int o = wave; o < MF * NF; o += 4) {
    const int m = o / NF, f = o % NF;
    if (m >= nmf) continue;
    floatx4 s = red[0][m * NFT + f][lane];
    floatx4 u = {0.f, 0.f, 0.f, 0.f};
    if (EPI == EPI_GEGLU_BF16) u = red[0][m * NFT + NF + f][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      s += red[w][m * NFT + f][lane];
      if (EPI == EPI_GEGLU_BF16) u += red[w][m * NFT + NF + f][lane];
    }
    const int col = n_base + f * 16 + lr;
    if (col >= g.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = m * 16 + lg * 4 + i;
      if (rl >= nrows) continue;
      const long off = (long)(r0 + rl) * g.ldc + col;
      const float v = s[i];
      if (EPI == EPI_STORE_BF16) {
        reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(v);
      } else if (EPI == EPI_STORE_F32) {
        reinterpret_cast<float*>(g.C)[(long)zk * g.c_kstride + off] = v;
      } else if (EPI == EPI_ADD_F32) {
        reinterpret_cast<float*>(g.C)[off] += v;
      } else if (EPI == EPI_ADD_GATED_F32) {
        reinterpret_cast<float*>(g.C)[off] += sigmoidf_(bf2f(g.col_gate[col])) * v;
      } else {
        reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(gelu_tanh(v) * u[i]);
      }
    }
  }
}

template <int EPI, int MF, int NF>
static hipError_t launch(const GemmArgs& a, hipStream_t s) {
  const int ntiles = (a.N + 16 * NF - 1) / (16 * NF);
  const long total = (long)a.items_max * ntiles * a.k_split;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<EPI, MF, NF>), dim3((unsigned)total), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t gemm(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.K % 32 != 0 || a.k_chunk % 32 != 0 || a.k_split < 1 || a.items_max < 1) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE_BF16: return launch<EPI_STORE_BF16, 4, 4>(a, s);
    case EPI_STORE_F32: return launch<EPI_STORE_F32, 4, 4>(a, s);
    case EPI_ADD_F32: return launch<EPI_ADD_F32, 4, 4>(a, s);
    case EPI_ADD_GATED_F32: return launch<EPI_ADD_GATED_F32, 4, 4>(a, s);
    case EPI_GEGLU_BF16: return launch<EPI_GEGLU_BF16, 4, 2>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
