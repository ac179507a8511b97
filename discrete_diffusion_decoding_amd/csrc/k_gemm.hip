// Weight-streaming bf16 GEMM on MFMA (v_mfma_f32_16x16x32_bf16) for gfx950.
//
// Every matrix product of the denoising step has few activation rows (256 canvas
// tokens, ~16 per expert) against a large weight matrix, so the kernels are
// built to stream each weight byte from HBM once:
//   * a workgroup (4 waves) owns a tile of 4*NF*16 weight rows (output columns);
//     each wave loads its own weight rows straight into MFMA B registers with
//     16-byte loads (no LDS round trip, two k-steps in flight per iteration);
//   * the activation rows (A) are small and re-read from L1/L2 by every wave;
//     expert rows are gathered through a row map instead of being copied;
//   * rows are taken in chunks of 16*MF; `m_split` spreads a large row count over
//     several workgroups that share a weight tile;
//   * the 1-D grid is ordered so that each XCD (workgroup id mod 8) walks a
//     contiguous range of (group, tile, row-chunk) items: the row-chunks of a
//     weight tile land on one XCD back to back and hit its L2.
#include "dg_kernels.hpp"

namespace dg {

template <int EPI, int MF, int NF>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  if (g.flag && *g.flag) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntiles = (g.N + 64 * NF - 1) / (64 * NF);
  const int nz = g.m_split * g.k_split;
  const long total = (long)g.G * ntiles * nz;
  // XCD-aware linearisation: workgroup b runs on XCD b % 8.
  const long b = blockIdx.x;
  const long q = total / 8, rr = total % 8;
  const long x = b % 8, j = b / 8;
  const long item = x * q + (x < rr ? x : rr) + j;
  if (item >= total) return;
  const int grp = (int)(item / ((long)ntiles * nz));
  const long rem = item % ((long)ntiles * nz);
  const int tile = (int)(rem / nz);
  const int z = (int)(rem % nz);
  const int zm = z % g.m_split, zk = z / g.m_split;

  int r0 = 0, r1 = g.M;
  if (g.group_off) {
    r0 = g.group_off[grp];
    r1 = g.group_off[grp + 1];
  }
  const int n_base = (tile * 4 + wave) * NF * 16;
  if (n_base >= g.N || r1 <= r0) return;
  const int kb = zk * g.k_chunk;
  const int ke = min(g.K, kb + g.k_chunk);

  const int lr = lane & 15, lg = lane >> 4;
  const bf16_t* W = g.W + (long)grp * g.w_gstride;
  const bf16_t* bp[NF];
  const bf16_t* bp2[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int n = min(n_base + f * 16 + lr, g.N - 1);
    bp[f] = W + (long)n * g.ldw + lg * 8;
    if (EPI == EPI_GEGLU_BF16) bp2[f] = g.W2 + (long)grp * g.w_gstride + (long)n * g.ldw + lg * 8;
  }

  constexpr int CH = 16 * MF;
  for (int rc = r0 + zm * CH; rc < r1; rc += g.m_split * CH) {
    const int nrows = min(CH, r1 - rc);
    const int nmf = (nrows + 15) >> 4;
    const bf16_t* ap[MF];
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      const int r = min(rc + m * 16 + lr, r1 - 1);
      const int ar = g.a_rows ? g.a_rows[r] : r;
      ap[m] = g.A + (long)ar * g.lda + lg * 8;
    }
    floatx4 acc[MF][NF];
    floatx4 acc2[MF][NF];
#pragma unroll
    for (int m = 0; m < MF; ++m)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        acc[m][f] = floatx4{0.f, 0.f, 0.f, 0.f};
        acc2[m][f] = floatx4{0.f, 0.f, 0.f, 0.f};
      }

    // software pipeline: weights for the next 64-wide k block are requested
    // before the MFMAs of the current block are issued
    bf16x8 wb[2][NF], wb2[2][NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      wb[0][f] = load_bf16x8(bp[f] + kb);
      wb[1][f] = load_bf16x8(bp[f] + kb + 32);
      if (EPI == EPI_GEGLU_BF16) {
        wb2[0][f] = load_bf16x8(bp2[f] + kb);
        wb2[1][f] = load_bf16x8(bp2[f] + kb + 32);
      }
    }
    for (int k = kb; k < ke; k += 64) {
      bf16x8 nb[2][NF], nb2[2][NF];
      const bool more = (k + 64) < ke;
      if (more) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          nb[0][f] = load_bf16x8(bp[f] + k + 64);
          nb[1][f] = load_bf16x8(bp[f] + k + 96);
          if (EPI == EPI_GEGLU_BF16) {
            nb2[0][f] = load_bf16x8(bp2[f] + k + 64);
            nb2[1][f] = load_bf16x8(bp2[f] + k + 96);
          }
        }
      }
      bf16x8 av[2][MF];
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        if (m < nmf) {
          av[0][m] = load_bf16x8(ap[m] + k);
          av[1][m] = load_bf16x8(ap[m] + k + 32);
        }
      }
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        if (m < nmf) {
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            acc[m][f] = mfma16x16x32(av[0][m], wb[0][f], acc[m][f]);
            acc[m][f] = mfma16x16x32(av[1][m], wb[1][f], acc[m][f]);
            if (EPI == EPI_GEGLU_BF16) {
              acc2[m][f] = mfma16x16x32(av[0][m], wb2[0][f], acc2[m][f]);
              acc2[m][f] = mfma16x16x32(av[1][m], wb2[1][f], acc2[m][f]);
            }
          }
        }
      }
      if (more) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          wb[0][f] = nb[0][f];
          wb[1][f] = nb[1][f];
          if (EPI == EPI_GEGLU_BF16) {
            wb2[0][f] = nb2[0][f];
            wb2[1][f] = nb2[1][f];
          }
        }
      }
    }

    // epilogue: lane holds rows 4*lg + i of each 16-row fragment, column lr
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      if (m >= nmf) continue;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int col = n_base + f * 16 + lr;
        if (col >= g.N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rc + m * 16 + lg * 4 + i;
          if (row >= rc + nrows) continue;
          const float v = acc[m][f][i];
          const long off = (long)row * g.ldc + col;
          if (EPI == EPI_STORE_BF16) {
            reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(v);
          } else if (EPI == EPI_STORE_F32) {
            reinterpret_cast<float*>(g.C)[(long)zk * g.c_kstride + off] = v;
          } else if (EPI == EPI_ADD_F32) {
            reinterpret_cast<float*>(g.C)[off] += v;
          } else if (EPI == EPI_ADD_GATED_F32) {
            reinterpret_cast<float*>(g.C)[off] += sigmoidf_(bf2f(g.col_gate[col])) * v;
          } else {  // GEGLU
            reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(gelu_tanh(v) * acc2[m][f][i]);
          }
        }
      }
    }
  }
}

template <int EPI, int MF, int NF>
static hipError_t launch(const GemmArgs& a, hipStream_t s) {
  const int ntiles = (a.N + 64 * NF - 1) / (64 * NF);
  const long total = (long)a.G * ntiles * a.m_split * a.k_split;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<EPI, MF, NF>), dim3((unsigned)total), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t gemm(int epi, int mf, const GemmArgs& a, hipStream_t s) {
  if (a.K % 64 != 0 || a.k_chunk % 64 != 0) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE_BF16: return launch<EPI_STORE_BF16, 4, 2>(a, s);
    case EPI_STORE_F32: return launch<EPI_STORE_F32, 4, 2>(a, s);
    case EPI_ADD_F32: return launch<EPI_ADD_F32, 4, 2>(a, s);
    case EPI_ADD_GATED_F32: return launch<EPI_ADD_GATED_F32, 4, 2>(a, s);
    case EPI_GEGLU_BF16: return launch<EPI_GEGLU_BF16, 4, 1>(a, s);
  }
  (void)mf;
  return hipErrorInvalidValue;
}

}  // namespace dg
