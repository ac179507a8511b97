// Weight-streaming bf16 GEMM on MFMA (v_mfma_f32_16x16x32_bf16) for gfx950.
//
// Every product of the denoising step pairs few activation rows (256 canvas
// tokens; ~16-100 per expert) with a large weight matrix, so the kernel is built
// to keep many weight bytes in flight and to read each byte once:
//   * a workgroup (4 waves) owns one output tile: <= 64 activation rows (one
//     "item": a chunk of one expert's rows, or of the dense rows) x 64 weight rows
//     (GEGLU: 32 gate rows and the 32 matching up rows);
//   * the tiles are streamed through a 4-stage ring of LDS buffers, 64 columns
//     per stage, with direct global->LDS loads (global_load_lds_dwordx4): every
//     load instruction moves 8 whole 128-byte rows, three stages (48 KB) are in
//     flight while the fourth is multiplied, and no registers hold staged data;
//   * 16-byte slots of each 128-byte LDS row are XOR-swizzled by (row mod 8) so
//     the MFMA operand reads (16 rows x 64 bytes per instruction) spread over
//     the banks;
//   * wave w multiplies weight rows 16w..16w+15 by all activation fragments;
//   * expert rows are gathered through a row map (no copies), large experts are
//     cut into several items on different workgroups, and a split-K mode writes
//     partial tiles for a later reduction.
// Synchronisation uses plain s_barrier (no memory fence, which would force
// every outstanding load to finish) plus an explicit vmcnt wait for the stage
// about to be read (s_waitcnt encoding on gfx9: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8]).
#include "dg_kernels.hpp"

namespace dg {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kStageElems = 2 * 64 * 64;  // A tile then B tile, 64 rows x 64 bf16 each

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) bf16_t S0[kStageElems];
  __shared__ __attribute__((aligned(1024))) bf16_t S1[kStageElems];
  __shared__ __attribute__((aligned(1024))) bf16_t S2[kStageElems];
  __shared__ __attribute__((aligned(1024))) bf16_t S3[kStageElems];
  if (g.flag && *g.flag) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr bool GEGLU = EPI == EPI_GEGLU_BF16;
  constexpr int NCOL = GEGLU ? 32 : 64;   // output columns per tile
  const int ntiles = (g.N + NCOL - 1) / NCOL;
  const long bidx = blockIdx.x;
  const int item = (int)(bidx % g.items_max);
  const long rest = bidx / g.items_max;
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
    r0 = item * 64;
    nrows = min(64, g.M - r0);
  }
  if (nrows <= 0) return;
  const int nmf = (nrows + 15) >> 4;
  const int n_base = tile * NCOL;
  const int kb = zk * g.k_chunk;
  const int ke = min(g.K, kb + g.k_chunk);
  const int nst = (ke - kb) >> 6;   // 64-column stages

  // ---- per-lane global addresses of this wave's DMA rows --------------------
  // wave w moves row groups 2w and 2w+1 (8 rows each) of both the A and the B
  // tile; lane l fills LDS slot l%8 of row l/8 with global 16-byte part
  // (l%8) ^ (row%8) of that row.
  const int lrow = lane >> 3, lslot = lane & 7;
  const int part = lslot ^ lrow;
  const bf16_t* asrc[2];
  const bf16_t* bsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (2 * wave + j) * 8 + lrow;       // 0..63
    const int ar_l = r0 + min(row, nrows - 1);
    const int ar = g.a_rows ? g.a_rows[ar_l] : ar_l;
    asrc[j] = g.A + (long)ar * g.lda + kb + part * 8;
    int wrow;
    const bf16_t* Wb;
    if (GEGLU) {
      wrow = min(n_base + (row & 31), g.N - 1);
      Wb = row < 32 ? g.W : g.W2;
    } else {
      wrow = min(n_base + row, g.N - 1);
      Wb = g.W;
    }
    bsrc[j] = Wb + (long)grp * g.w_gstride + (long)wrow * g.ldw + kb + part * 8;
  }
  const int dst_a = (2 * wave) * 8 * 64;              // element offset of this wave's first A row group
  const int dst_b = 64 * 64 + dst_a;

#define DG_ISSUE(S, ST)                                                                          \
  do {                                                                                           \
    const int co_ = (ST) << 6;                                                                   \
    __builtin_amdgcn_global_load_lds((const void*)(asrc[0] + co_), (lds_void_t*)&S[dst_a], 16, 0, 0);       \
    __builtin_amdgcn_global_load_lds((const void*)(asrc[1] + co_), (lds_void_t*)&S[dst_a + 512], 16, 0, 0); \
    __builtin_amdgcn_global_load_lds((const void*)(bsrc[0] + co_), (lds_void_t*)&S[dst_b], 16, 0, 0);       \
    __builtin_amdgcn_global_load_lds((const void*)(bsrc[1] + co_), (lds_void_t*)&S[dst_b + 512], 16, 0, 0); \
  } while (0)

  // ---- MFMA operand reads ------------------------------------------------------
  const int lr = lane & 15, lg = lane >> 4;
  const int brow = 16 * wave + lr;                    // weight row in the B tile
  floatx4 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};

#define DG_COMPUTE(S)                                                                            \
  do {                                                                                           \
    _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                              \
      const int p_ = 4 * j + lg;                                                                 \
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(&S[64 * 64 + brow * 64 + ((p_ ^ (brow & 7)) << 3)]); \
      bf16x8 af[4];                                                                              \
      _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                            \
        const int arow = 16 * m + lr;                                                            \
        af[m] = *reinterpret_cast<const bf16x8*>(&S[arow * 64 + ((p_ ^ (arow & 7)) << 3)]);      \
      }                                                                                          \
      _Pragma("unroll") for (int m = 0; m < 4; ++m) acc[m] = mfma16x16x32(af[m], bf, acc[m]);    \
    }                                                                                            \
  } while (0)

  // Every stage issues its loads unconditionally (stage index clamped to the
  // last one: the surplus loads land in a buffer that is not read again), so
  // exactly two younger stages (8 loads per lane) are pending when a stage is
  // read and one constant wait suffices.
#define DG_ITER(SI, CUR, NXT)                                                                    \
  do {                                                                                           \
    const int s_ = (SI);                                                                         \
    __builtin_amdgcn_s_waitcnt((8 & 0xF) | (0x7 << 4) | (0xF << 8));                             \
    __builtin_amdgcn_s_barrier();                                                                \
    DG_ISSUE(NXT, min(s_ + 3, nst - 1));                                                         \
    DG_COMPUTE(CUR);                                                                             \
  } while (0)

  if (nst > 0) {
    DG_ISSUE(S0, 0);
    DG_ISSUE(S1, min(1, nst - 1));
    DG_ISSUE(S2, min(2, nst - 1));
    int s = 0;
    for (; s + 4 <= nst; s += 4) {
      DG_ITER(s, S0, S3);
      DG_ITER(s + 1, S1, S0);
      DG_ITER(s + 2, S2, S1);
      DG_ITER(s + 3, S3, S2);
    }
    if (s < nst) DG_ITER(s, S0, S3);
    if (s + 1 < nst) DG_ITER(s + 1, S1, S0);
    if (s + 2 < nst) DG_ITER(s + 2, S2, S1);
  }
#undef DG_ISSUE
#undef DG_COMPUTE
#undef DG_ITER

  // ---- epilogue ------------------------------------------------------------------
  // lane holds rows 4*lg + i of each 16-row fragment, column lr of the wave's 16
  if (GEGLU) {
    // waves 2,3 hold the up projections of the columns of waves 0,1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    floatx4* red = reinterpret_cast<floatx4*>(S0);
    if (wave >= 2) {
#pragma unroll
      for (int m = 0; m < 4; ++m) red[((wave - 2) * 4 + m) * 64 + lane] = acc[m];
    }
    __syncthreads();
    if (wave >= 2) return;
  }
  const int col = n_base + 16 * wave + lr;
  if (col >= g.N) return;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m >= nmf) continue;
    floatx4 u = {0.f, 0.f, 0.f, 0.f};
    if (GEGLU) u = reinterpret_cast<floatx4*>(S0)[(wave * 4 + m) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = 16 * m + 4 * lg + i;
      if (rl >= nrows) continue;
      const long off = (long)(r0 + rl) * g.ldc + col;
      const float v = acc[m][i];
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

template <int EPI>
static hipError_t launch(const GemmArgs& a, hipStream_t s) {
  constexpr int NCOL = (EPI == EPI_GEGLU_BF16) ? 32 : 64;
  const int ntiles = (a.N + NCOL - 1) / NCOL;
  const long total = (long)a.items_max * ntiles * a.k_split;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<EPI>), dim3((unsigned)total), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t gemm(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.K % 64 != 0 || a.k_chunk % 64 != 0 || a.k_split < 1 || a.items_max < 1) return hipErrorInvalidValue;
  if (a.lda % 8 != 0 || a.ldw % 8 != 0) return hipErrorInvalidValue;   // 16-byte aligned rows
  switch (epi) {
    case EPI_STORE_BF16: return launch<EPI_STORE_BF16>(a, s);
    case EPI_STORE_F32: return launch<EPI_STORE_F32>(a, s);
    case EPI_ADD_F32: return launch<EPI_ADD_F32>(a, s);
    case EPI_ADD_GATED_F32: return launch<EPI_ADD_GATED_F32>(a, s);
    case EPI_GEGLU_BF16: return launch<EPI_GEGLU_BF16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
