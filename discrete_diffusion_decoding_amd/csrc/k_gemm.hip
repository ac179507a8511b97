// Weight-streaming bf16 GEMM on MFMA (v_mfma_f32_16x16x32_bf16) for gfx950.
//
// Every product of the denoising step pairs few activation rows (256 canvas
// tokens; ~16-100 per expert) with a large weight matrix, so the kernel is built
// to keep many weight bytes in flight and to read each byte once:
//   * a workgroup (4 waves) owns one output tile: <= 64 activation rows (one
//     "item": a chunk of one expert's rows, or of the dense rows; dense products
//     may take 128) x 64 or 128 weight rows (GEGLU: half gate rows, half the
//     matching up rows);
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

#include <type_traits>

namespace dg {

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate (gfx9 layout): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt_hi[15:14]; only the vector-memory count is waited for.
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Cache policy of the weight loads.  A weight tile that one workgroup alone
// reads is loaded non-temporal (the nt bit of the load's cache-policy operand):
// the L2 then gives its lines up first and keeps the activation tiles, which
// every weight tile of the product re-reads.  A tile that several row chunks
// share (dense products over more rows than one tile, experts of several
// chunks) keeps the default policy, so the chunks that follow hit in L2.
constexpr int kPolicyStream = 2;
#define DG_LDS_LOAD(SRC, DST, NT)                                                              \
  do {                                                                                         \
    if (NT) __builtin_amdgcn_global_load_lds((const void*)(SRC), (lds_void_t*)(DST), 16, 0, kPolicyStream); \
    else __builtin_amdgcn_global_load_lds((const void*)(SRC), (lds_void_t*)(DST), 16, 0, 0);   \
  } while (0)

// ITEMS: rows come from the expert work list (grouped expert products);
// otherwise dense rows in AR-row chunks.  AR: activation rows per tile (32 or
// 64).  BW: weight rows per tile (64 or 128; each of the 4 waves multiplies BW/4
// of them by all AR activation rows).  NS: depth of the LDS ring (NS - 1
// stages in flight).  The weight stream is what the product is bound by; the
// activation tile is re-read from L2 for every weight tile, so a wider BW
// spends fewer DMA and LDS cycles per weight byte.
// workgroups per CU a variant is built for: as many as its ring fits in the
// 160 KB of LDS, at most two (three for double-buffered rings)
template <int AR, int BW, int NS>
constexpr int gemm_wg_per_cu() {
  return NS * (AR + BW) * 128 > 80 * 1024 ? 1 : (NS == 2 && (AR + BW) * 128 * NS <= 53 * 1024 ? 3 : 2);
}

template <int EPI, bool ITEMS, int AR, int BW, int NS>
__global__ __launch_bounds__(256, (gemm_wg_per_cu<AR, BW, NS>())) void gemm_kernel(GemmArgs g) {
  static_assert(AR == 32 || AR == 64 || (AR == 128 && !ITEMS), "activation tile of 32, 64 (or dense 128) rows");
  static_assert(BW == 64 || BW == 128, "weight tile of 64 or 128 rows");
  static_assert(NS >= 2 && NS <= 6, "ring of 2..6 stages");
  constexpr int SE = (AR + BW) * 64;         // stage: AR activation rows then BW weight rows, 64 bf16 each
  constexpr int NG = (AR + BW) / 8;          // 8-row groups per stage (one 1 KB DMA each)
  constexpr int GPW = NG / 4;                // groups per wave
  constexpr int NAF = AR / 16;               // activation fragments
  constexpr int WPW = BW / 4;                // weight rows per wave
  constexpr int NBF = WPW / 16;              // weight fragments per wave
  static_assert(NG % 4 == 0, "groups split evenly over 4 waves");
  static_assert(NS * SE * 2 * gemm_wg_per_cu<AR, BW, NS>() <= 160 * 1024, "the ring fits the LDS of a CU");
  __shared__ __attribute__((aligned(1024))) bf16_t S0[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S1[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S2[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S3[NS > 3 ? SE : 1];
  __shared__ __attribute__((aligned(1024))) bf16_t S4[NS > 4 ? SE : 1];
  __shared__ __attribute__((aligned(1024))) bf16_t S5[NS > 5 ? SE : 1];
  if (g.flag && *g.flag) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr bool GEGLU = EPI == EPI_GEGLU_BF16;
  constexpr int NCOL = GEGLU ? BW / 2 : BW;   // output columns per tile
  const int ntiles = (g.N + NCOL - 1) / NCOL;
  int item, tile, zk;
  bool wnt;
  if (ITEMS) {
    // XCD x (blocks b with b % 8 == x) takes the x-th eighth of the actual
    // (item, tile) units, tile-major within an item, so the gathered
    // activation rows of an item are fetched into one (at most two) XCD's L2
    // and every XCD gets the same number of units (to one)
    const long per = (long)ntiles * g.k_split;
    const long nu = (long)(*g.n_items) * per;
    const int x = blockIdx.x & 7;
    const long w = blockIdx.x >> 3;
    const long lo = (x * nu) >> 3, hi = ((x + 1) * nu) >> 3;
    if (w >= hi - lo) return;
    const long u = lo + w;
    item = (int)(u / per);
    long rest = u % per;
    {
      // an expert of several 64-row chunks (items.w = chunk index << 16 |
      // chunk count): its units run chunk-fastest, so consecutive workgroups
      // of one XCD share each weight tile
      const int wv = g.items[item].w;
      const int ci = wv >> 16, ce = wv & 0xFFFF;
      wnt = __builtin_amdgcn_readfirstlane(ce) == 1;
      if (ce > 1) {
        const long p = (long)ci * per + rest;
        item = item - ci + (int)(p % ce);
        rest = p / ce;
      }
    }
    tile = (int)(rest % ntiles);
    zk = (int)(rest / ntiles);
  } else {
    const long bidx = xcd_logical_block((long)g.items_max * ntiles * g.k_split);
    if (bidx < 0) return;
    item = (int)(bidx % g.items_max);
    const long rest = bidx / g.items_max;
    tile = (int)(rest % ntiles);
    zk = (int)(rest / ntiles);
    wnt = g.items_max == 1;
  }

  int grp, r0, nrows;
  if (ITEMS) {
    if (item >= *g.n_items) return;
    const int4 it = g.items[item];
    grp = it.x;
    r0 = it.y;
    nrows = it.z;
  } else {
    grp = 0;
    r0 = item * AR;
    nrows = min(AR, g.M - r0);
  }
  if (nrows <= 0) return;
  const int n_base = tile * NCOL;
  const int kb = zk * g.k_chunk;
  const int ke = min(g.K, kb + g.k_chunk);
  const int nst = (ke - kb) >> 6;   // 64-column stages

  // ---- per-lane global addresses of this wave's DMA rows --------------------
  // the stage's 8-row groups (activation groups first, then weight groups) are
  // dealt to the waves in turn: wave w moves groups w, w+4, ...; lane l fills
  // LDS slot l%8 of row l/8 of its group with global 16-byte part (l%8)^(row%8).
  // GEGLU tiles hold NCOL gate rows, then the NCOL matching up rows.
  const int lrow = lane >> 3, lslot = lane & 7;
  const int part = lslot ^ lrow;
  const bf16_t* src[GPW];
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    const int gi = wave + 4 * j;
    if (gi < AR / 8) {
      const int row = gi * 8 + lrow;
      const int ar_l = r0 + min(row, nrows - 1);
      const int ar = g.a_rows ? g.a_rows[ar_l] : ar_l;
      src[j] = g.A + (long)ar * g.lda + kb + part * 8;
    } else {
      const int row = (gi - AR / 8) * 8 + lrow;   // 0..BW-1
      int wrow;
      const bf16_t* Wb;
      if (GEGLU) {
        wrow = min(n_base + (row % NCOL), g.N - 1);
        Wb = row < NCOL ? g.W : g.W2;
      } else {
        wrow = min(n_base + row, g.N - 1);
        Wb = g.W;
      }
      src[j] = Wb + (long)grp * g.w_gstride + (long)wrow * g.ldw + kb + part * 8;
    }
  }

#define DG_ISSUE(S, ST)                                                                          \
  do {                                                                                           \
    const int co_ = (ST) << 6;                                                                   \
    _Pragma("unroll") for (int j = 0; j < GPW; ++j) {                                            \
      DG_LDS_LOAD(src[j] + co_, &S[(wave + 4 * j) * 512], j >= AR / 32 && kNT);                 \
    }                                                                                            \
  } while (0)

  // ---- MFMA operand reads ------------------------------------------------------
  const int lr = lane & 15, lg = lane >> 4;
  // weight-row offsets computed once: derived inside the read macro, the
  // compiler lost track of which LDS array a read targets and made it wait for
  // every DMA in flight
  int boff[NBF];
#pragma unroll
  for (int n = 0; n < NBF; ++n) boff[n] = AR * 64 + (WPW * wave + 16 * n + lr) * 64;
  floatx4 acc[NAF][NBF];
#pragma unroll
  for (int m = 0; m < NAF; ++m)
#pragma unroll
    for (int n = 0; n < NBF; ++n) acc[m][n] = floatx4{0.f, 0.f, 0.f, 0.f};

#define DG_READ(S)                                                                               \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                                \
    const int p_ = 4 * j + lg;                                                                   \
    _Pragma("unroll") for (int n = 0; n < NBF; ++n)                                              \
      bf[j][n] = *reinterpret_cast<const bf16x8*>(&S[boff[n] + ((p_ ^ (lr & 7)) << 3)]);         \
    _Pragma("unroll") for (int m = 0; m < NAF; ++m) {                                            \
      const int arow = 16 * m + lr;                                                              \
      af[j][m] = *reinterpret_cast<const bf16x8*>(&S[arow * 64 + ((p_ ^ (arow & 7)) << 3)]);     \
    }                                                                                            \
  }
#define DG_MMA()                                                                                 \
  _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                  \
    _Pragma("unroll") for (int m = 0; m < NAF; ++m)                                              \
      _Pragma("unroll") for (int n = 0; n < NBF; ++n) acc[m][n] = mfma16x16x32(af[j][m], bf[j][n], acc[m][n]);

  // Every stage issues its loads unconditionally (stage index clamped to the
  // last one: the surplus loads land in a buffer that is not read again), so
  // exactly NS - 2 younger stages are pending when a stage is read and one
  // constant wait suffices.  The stage's LDS reads precede the next DMA issue
  // (sched_barrier), so the compiler adds no wait of its own.
#define DG_ITER(SI, CUR, NXT)                                                                    \
  do {                                                                                           \
    const int s_ = (SI);                                                                         \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * GPW));                                      \
    __builtin_amdgcn_s_barrier();                                                                \
    DG_READ(CUR);                                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    DG_ISSUE(NXT, min(s_ + NS - 1, nst - 1));                                                    \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    DG_MMA();                                                                                    \
  } while (0)
  // after the last full round every stage has been issued: the remaining
  // stages only drain the ring (the first wait covers all of them)
#define DG_TAIL(CUR)                                                                             \
  do {                                                                                           \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                                                   \
    __builtin_amdgcn_s_barrier();                                                                \
    DG_READ(CUR);                                                                                \
    DG_MMA();                                                                                    \
  } while (0)
  bf16x8 af[2][NAF], bf[2][NBF];

  // the pipeline is built twice, with and without the streaming policy on
  // the weight loads (an immediate of the load instruction)
  auto pipeline = [&](auto nt_tag) {
    constexpr bool kNT = decltype(nt_tag)::value;
    DG_ISSUE(S0, 0);
    if (NS > 2) DG_ISSUE(S1, min(1, nst - 1));
    if (NS > 3) DG_ISSUE(S2, min(2, nst - 1));
    if (NS > 4) DG_ISSUE(S3, min(3, nst - 1));
    if (NS > 5) DG_ISSUE(S4, min(4, nst - 1));
    int s = 0;
    if (NS == 2) {
      for (; s + 2 <= nst; s += 2) {
        DG_ITER(s, S0, S1); DG_ITER(s + 1, S1, S0);
      }
      if (s < nst) DG_TAIL(S0);
    } else if (NS == 3) {
      for (; s + 3 <= nst; s += 3) {
        DG_ITER(s, S0, S2); DG_ITER(s + 1, S1, S0); DG_ITER(s + 2, S2, S1);
      }
      if (s < nst) DG_TAIL(S0);
      if (s + 1 < nst) DG_TAIL(S1);
    } else if (NS == 4) {
      for (; s + 4 <= nst; s += 4) {
        DG_ITER(s, S0, S3); DG_ITER(s + 1, S1, S0); DG_ITER(s + 2, S2, S1); DG_ITER(s + 3, S3, S2);
      }
      if (s < nst) DG_TAIL(S0);
      if (s + 1 < nst) DG_TAIL(S1);
      if (s + 2 < nst) DG_TAIL(S2);
    } else if (NS == 5) {
      for (; s + 5 <= nst; s += 5) {
        DG_ITER(s, S0, S4); DG_ITER(s + 1, S1, S0); DG_ITER(s + 2, S2, S1); DG_ITER(s + 3, S3, S2);
        DG_ITER(s + 4, S4, S3);
      }
      if (s < nst) DG_TAIL(S0);
      if (s + 1 < nst) DG_TAIL(S1);
      if (s + 2 < nst) DG_TAIL(S2);
      if (s + 3 < nst) DG_TAIL(S3);
    } else {
      for (; s + 6 <= nst; s += 6) {
        DG_ITER(s, S0, S5); DG_ITER(s + 1, S1, S0); DG_ITER(s + 2, S2, S1); DG_ITER(s + 3, S3, S2);
        DG_ITER(s + 4, S4, S3); DG_ITER(s + 5, S5, S4);
      }
      if (s < nst) DG_TAIL(S0);
      if (s + 1 < nst) DG_TAIL(S1);
      if (s + 2 < nst) DG_TAIL(S2);
      if (s + 3 < nst) DG_TAIL(S3);
      if (s + 4 < nst) DG_TAIL(S4);
    }
  };
  if (nst > 0) {
    if (wnt) pipeline(std::true_type{});
    else pipeline(std::false_type{});
  }
#undef DG_TAIL
#undef DG_ISSUE
#undef DG_READ
#undef DG_MMA
#undef DG_ITER

  // ---- epilogue ------------------------------------------------------------------
  // lane holds rows 4*lg + i of each 16-row fragment, column lr of each of the
  // wave's 16-column fragments
  if (GEGLU) {
    // waves 2,3 hold the up projections of the columns of waves 0,1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    floatx4* red = reinterpret_cast<floatx4*>(S0);
    if (wave >= 2) {
#pragma unroll
      for (int m = 0; m < NAF; ++m)
#pragma unroll
        for (int n = 0; n < NBF; ++n) red[(((wave - 2) * NAF + m) * NBF + n) * 64 + lane] = acc[m][n];
    }
    __syncthreads();
    if (wave >= 2) return;
  }
#pragma unroll
  for (int n = 0; n < NBF; ++n) {
    const int col = n_base + WPW * wave + 16 * n + lr;
    if (col >= g.N) continue;
#pragma unroll
    for (int m = 0; m < NAF; ++m) {
      floatx4 u = {0.f, 0.f, 0.f, 0.f};
      if (GEGLU) u = reinterpret_cast<floatx4*>(S0)[((wave * NAF + m) * NBF + n) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 16 * m + 4 * lg + i;
        if (rl >= nrows) continue;
        const long off = (long)(r0 + rl) * g.ldc + col;
        const float v = acc[m][n][i];
        if (EPI == EPI_STORE_BF16) {
          reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(v);
        } else if (EPI == EPI_STORE_F32) {
          reinterpret_cast<float*>(g.C)[(long)zk * g.c_kstride + off] = v;
        } else {
          reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(gelu_tanh(v) * u[i]);
        }
      }
    }
  }
}

template <int EPI, bool ITEMS, int AR, int BW, int NS>
static hipError_t launch_v(GemmArgs a, hipStream_t s) {
  constexpr int NCOL = (EPI == EPI_GEGLU_BF16) ? BW / 2 : BW;
  if (!ITEMS) a.items_max = (a.M + AR - 1) / AR;
  const int ntiles = (a.N + NCOL - 1) / NCOL;
  // work lists: every XCD gets room for an eighth of items_max (rounded up)
  const long total = (ITEMS ? 8L * ((a.items_max + 7) / 8) : (long)a.items_max) * ntiles * a.k_split;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<EPI, ITEMS, AR, BW, NS>), dim3(xcd_grid(total)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dense store products on 8 waves (two per SIMD).  With one workgroup of 4
// waves per CU (the 256 tiles of a 256-row projection), a stage's LDS reads run
// at the latency-bound rate of 4 waves and each SIMD's MFMA chains wait on
// them; 8 waves read LDS faster and a SIMD's two waves overlap one's reads with
// the other's MFMAs.  The waves form a 2 x 4 grid: wave w multiplies activation
// rows (AR / 2) (w / 4) .. + AR / 2 - 1 by weight rows (BW / 4) (w % 4) ..
// + BW / 4 - 1, so each wave reads half of the stage's activation tile and a
// quarter of its weight tile.  Ring, swizzle, DMA and waits as gemm_kernel.
template <int AR, int BW, int NS>
constexpr int gemm8_wg_per_cu() {
  return NS * (AR + BW) * 128 > 80 * 1024 ? 1 : 2;
}

template <int EPI, int AR, int BW, int NS>
__global__ __launch_bounds__(512, (gemm8_wg_per_cu<AR, BW, NS>())) void gemm8_kernel(GemmArgs g) {
  static_assert(EPI == EPI_STORE_BF16 || EPI == EPI_STORE_F32, "plain stores");
  static_assert(AR == 64 || AR == 128, "activation tile of 64 or 128 rows");
  static_assert(BW == 64 || BW == 128, "weight tile of 64 or 128 rows");
  static_assert(NS >= 2 && NS <= 5, "ring of 2..5 stages");
  constexpr int SE = (AR + BW) * 64;   // stage: AR activation rows then BW weight rows, 64 bf16 each
  constexpr int NG = (AR + BW) / 8;    // 8-row groups per stage (one 1 KB DMA each)
  constexpr int GPW = NG / 8;          // groups per wave
  constexpr int NAF = AR / 32;         // activation fragments per wave (half the tile)
  constexpr int WPW = BW / 4;          // weight rows per wave
  constexpr int NBF = WPW / 16;        // weight fragments per wave
  static_assert(NG % 8 == 0 && (AR / 8) % 8 == 0, "groups split evenly over 8 waves, activation groups first");
  static_assert(NS * SE * 2 * gemm8_wg_per_cu<AR, BW, NS>() <= 160 * 1024, "the ring fits the LDS of a CU");
  __shared__ __attribute__((aligned(1024))) bf16_t S0[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S1[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S2[NS > 2 ? SE : 1];
  __shared__ __attribute__((aligned(1024))) bf16_t S3[NS > 3 ? SE : 1];
  __shared__ __attribute__((aligned(1024))) bf16_t S4[NS > 4 ? SE : 1];
  if (g.flag && *g.flag) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int ntiles = (g.N + BW - 1) / BW;
  const long bidx = xcd_logical_block((long)g.items_max * ntiles * g.k_split);
  if (bidx < 0) return;
  const int item = (int)(bidx % g.items_max);
  const long rest = bidx / g.items_max;
  const int tile = (int)(rest % ntiles);
  const int zk = (int)(rest / ntiles);
  const bool wnt = g.items_max == 1;   // each weight tile is read by this workgroup only
  const int r0 = item * AR;
  const int nrows = min(AR, g.M - r0);
  if (nrows <= 0) return;
  const int n_base = tile * BW;
  const int kb = zk * g.k_chunk;
  const int ke = min(g.K, kb + g.k_chunk);
  const int nst = (ke - kb) >> 6;

  // DMA rows: wave w moves groups w, w + 8, ...; lane l fills LDS slot l % 8
  // of row l / 8 of its group with global 16-byte part (l % 8) ^ (row % 8)
  const int lrow = lane >> 3, lslot = lane & 7;
  const int part = lslot ^ lrow;
  const bf16_t* src[GPW];
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    const int gi = wave + 8 * j;
    if (j < AR / 64) {   // gi < AR / 8: activation rows
      const int row = gi * 8 + lrow;
      src[j] = g.A + (long)(r0 + min(row, nrows - 1)) * g.lda + kb + part * 8;
    } else {
      const int row = (gi - AR / 8) * 8 + lrow;
      src[j] = g.W + (long)min(n_base + row, g.N - 1) * g.ldw + kb + part * 8;
    }
  }
#define DG_ISSUE8(S, ST)                                                                         \
  do {                                                                                           \
    const int co_ = (ST) << 6;                                                                   \
    _Pragma("unroll") for (int j = 0; j < GPW; ++j)                                              \
      DG_LDS_LOAD(src[j] + co_, &S[(wave + 8 * j) * 512], j >= AR / 64 && kNT);                  \
  } while (0)

  const int lr = lane & 15, lg = lane >> 4;
  int aoff[NAF], boff[NBF];
#pragma unroll
  for (int m = 0; m < NAF; ++m) {
    const int arow = (AR / 2) * wm + 16 * m + lr;
    aoff[m] = arow * 64;
  }
#pragma unroll
  for (int n = 0; n < NBF; ++n) boff[n] = AR * 64 + (WPW * wn + 16 * n + lr) * 64;
  floatx4 acc[NAF][NBF];
#pragma unroll
  for (int m = 0; m < NAF; ++m)
#pragma unroll
    for (int n = 0; n < NBF; ++n) acc[m][n] = floatx4{0.f, 0.f, 0.f, 0.f};
  bf16x8 af[2][NAF], bf[2][NBF];
  // activation row (AR / 2) wm + 16 m + lr has row % 8 == lr % 8 (AR / 2 and 16 are multiples of 8)
#define DG_READ8(S)                                                                              \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                                \
    const int p_ = 4 * j + lg;                                                                   \
    _Pragma("unroll") for (int n = 0; n < NBF; ++n)                                              \
      bf[j][n] = *reinterpret_cast<const bf16x8*>(&S[boff[n] + ((p_ ^ (lr & 7)) << 3)]);         \
    _Pragma("unroll") for (int m = 0; m < NAF; ++m)                                              \
      af[j][m] = *reinterpret_cast<const bf16x8*>(&S[aoff[m] + ((p_ ^ (lr & 7)) << 3)]);         \
  }
#define DG_MMA8()                                                                                \
  _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                  \
    _Pragma("unroll") for (int m = 0; m < NAF; ++m)                                              \
      _Pragma("unroll") for (int n = 0; n < NBF; ++n) acc[m][n] = mfma16x16x32(af[j][m], bf[j][n], acc[m][n]);
#define DG_ITER8(SI, CUR, NXT)                                                                   \
  do {                                                                                           \
    const int s_ = (SI);                                                                         \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * GPW));                                      \
    __builtin_amdgcn_s_barrier();                                                                \
    DG_READ8(CUR);                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    DG_ISSUE8(NXT, min(s_ + NS - 1, nst - 1));                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    DG_MMA8();                                                                                   \
  } while (0)
#define DG_TAIL8(CUR)                                                                            \
  do {                                                                                           \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                                                   \
    __builtin_amdgcn_s_barrier();                                                                \
    DG_READ8(CUR);                                                                               \
    DG_MMA8();                                                                                   \
  } while (0)
  auto pipeline = [&](auto nt_tag) {
    constexpr bool kNT = decltype(nt_tag)::value;
    DG_ISSUE8(S0, 0);
    if (NS > 2) DG_ISSUE8(S1, min(1, nst - 1));
    if (NS > 3) DG_ISSUE8(S2, min(2, nst - 1));
    if (NS > 4) DG_ISSUE8(S3, min(3, nst - 1));
    int s = 0;
    if (NS == 2) {
      for (; s + 2 <= nst; s += 2) {
        DG_ITER8(s, S0, S1); DG_ITER8(s + 1, S1, S0);
      }
      if (s < nst) DG_TAIL8(S0);
    } else if (NS == 3) {
      for (; s + 3 <= nst; s += 3) {
        DG_ITER8(s, S0, S2); DG_ITER8(s + 1, S1, S0); DG_ITER8(s + 2, S2, S1);
      }
      if (s < nst) DG_TAIL8(S0);
      if (s + 1 < nst) DG_TAIL8(S1);
    } else if (NS == 4) {
      for (; s + 4 <= nst; s += 4) {
        DG_ITER8(s, S0, S3); DG_ITER8(s + 1, S1, S0); DG_ITER8(s + 2, S2, S1); DG_ITER8(s + 3, S3, S2);
      }
      if (s < nst) DG_TAIL8(S0);
      if (s + 1 < nst) DG_TAIL8(S1);
      if (s + 2 < nst) DG_TAIL8(S2);
    } else {
      for (; s + 5 <= nst; s += 5) {
        DG_ITER8(s, S0, S4); DG_ITER8(s + 1, S1, S0); DG_ITER8(s + 2, S2, S1); DG_ITER8(s + 3, S3, S2);
        DG_ITER8(s + 4, S4, S3);
      }
      if (s < nst) DG_TAIL8(S0);
      if (s + 1 < nst) DG_TAIL8(S1);
      if (s + 2 < nst) DG_TAIL8(S2);
      if (s + 3 < nst) DG_TAIL8(S3);
    }
  };
  if (nst > 0) {
    if (wnt) pipeline(std::true_type{});
    else pipeline(std::false_type{});
  }
  __builtin_amdgcn_s_waitcnt(0);   // no DMA into LDS outlives the loop
#undef DG_TAIL8
#undef DG_ISSUE8
#undef DG_READ8
#undef DG_MMA8
#undef DG_ITER8

#pragma unroll
  for (int n = 0; n < NBF; ++n) {
    const int col = n_base + WPW * wn + 16 * n + lr;
    if (col >= g.N) continue;
#pragma unroll
    for (int m = 0; m < NAF; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = (AR / 2) * wm + 16 * m + 4 * lg + i;
        if (rl >= nrows) continue;
        const long off = (long)(r0 + rl) * g.ldc + col;
        if (EPI == EPI_STORE_BF16) reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(acc[m][n][i]);
        else reinterpret_cast<float*>(g.C)[(long)zk * g.c_kstride + off] = acc[m][n][i];
      }
    }
  }
}

template <int EPI, int AR, int BW, int NS>
static hipError_t launch_v8(GemmArgs a, hipStream_t s) {
  a.items_max = (a.M + AR - 1) / AR;
  const long total = (long)a.items_max * ((a.N + BW - 1) / BW) * a.k_split;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm8_kernel<EPI, AR, BW, NS>), dim3(xcd_grid(total)), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch8(const GemmArgs& a, hipStream_t s) {
  switch (a.tile_rows * 10000 + a.tile_cols * 10 + a.ring) {
    case 640644: return launch_v8<EPI, 64, 64, 4>(a, s);
    case 641283: return launch_v8<EPI, 64, 128, 3>(a, s);
    case 1280643: return launch_v8<EPI, 128, 64, 3>(a, s);
    case 1281283: return launch_v8<EPI, 128, 128, 3>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// variant chosen by the caller: a.tile_rows (activation rows), a.tile_cols
// (weight rows), a.ring (LDS ring depth)
template <int EPI, bool ITEMS>
static hipError_t launch(const GemmArgs& a, hipStream_t s) {
  if (a.tile_rows == 128) {
    if (ITEMS) return hipErrorInvalidValue;
    switch (a.tile_cols * 10 + a.ring) {
      case 643: return launch_v<EPI, false, 128, 64, 3>(a, s);
      case 1282: return launch_v<EPI, false, 128, 128, 2>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.tile_rows != 64) return hipErrorInvalidValue;
  const int v = a.tile_cols * 10 + a.ring;
  switch (v) {
    case 644: return launch_v<EPI, ITEMS, 64, 64, 4>(a, s);
    case 645: return launch_v<EPI, ITEMS, 64, 64, 5>(a, s);
    case 1283: return launch_v<EPI, ITEMS, 64, 128, 3>(a, s);
    case 1282: return launch_v<EPI, ITEMS, 64, 128, 2>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Few-row products (decoding: one activation row per sequence, a handful per
// expert).  The MFMA tile would spend 64 activation rows of DMA and LDS on each
// live row, so these stream the weights straight into registers instead: the
// item's activation rows (<= RB, its k chunk) are staged once in LDS, and a
// wave takes 8 weight rows, read 8 x 128 contiguous bytes per load
// instruction (lane l: row l / 8, 16-byte part l % 8 of each 128-byte step).
// KW waves share the same 8 rows and split the k steps into KW contiguous
// ranges of at most 16 steps, each issued as one batch of loads, so a wave
// makes about one round trip to memory (KW = 1, 2, 4 for slices of up to 16,
// 32, 64+ steps).  Lanes accumulate bf16 pair products in fp32
// (v_dot2_f32_bf16); the 8 lanes of a row are summed by shuffles and the KW
// waves through LDS.  Units are (item, column tile, k slice), as in the MFMA
// kernel, with the same epilogues (GEGLU: 4 gate rows and their 4 up rows per
// row set).
template <int KW>
constexpr int gemv_cols(bool geglu) { return (geglu ? 4 : 8) * (4 / KW); }
template <int EPI, bool ITEMS, int RB, int KW>
__global__ __launch_bounds__(256) void gemv_kernel(GemmArgs g) {
  constexpr bool GEGLU = EPI == EPI_GEGLU_BF16;
  constexpr int NCOL = gemv_cols<KW>(GEGLU);   // output columns per workgroup
  constexpr int U = 16;                        // 128-byte steps per batch of loads
  __shared__ __attribute__((aligned(16))) bf16_t X[RB * kGemvK];
  __shared__ float red[4][8][RB];
  if (g.flag && *g.flag) return;
  const int ntiles = (g.N + NCOL - 1) / NCOL;
  const long per = (long)ntiles * g.k_split;
  const long nunits = (ITEMS ? (long)*g.n_items : 1L) * per;
  const long u = blockIdx.x;
  if (u >= nunits) return;
  const int item = (int)(u / per);
  const int tile = (int)((u % per) % ntiles), zk = (int)((u % per) / ntiles);
  int grp, r0, nrows;
  if (ITEMS) {
    const int4 it = g.items[item];
    grp = it.x;
    r0 = it.y;
    nrows = min(it.z, RB);
  } else {
    grp = 0;
    r0 = 0;
    nrows = min(g.M, RB);
  }
  if (nrows <= 0) return;
  const int kb = zk * g.k_chunk;
  const int nk = min(g.K, kb + g.k_chunk) - kb;   // a multiple of 64
  if (nk <= 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int rs = lane >> 3, part = lane & 7;
  const int set = wave / KW, kw = wave % KW;   // row set of this wave, and its k range
  const int col = tile * NCOL + set * (GEGLU ? 4 : 8) + (GEGLU ? (rs & 3) : rs);
  const bool alt = ITEMS && g.Wx && grp >= g.grp_x;
  const bf16_t* Wb = alt ? ((GEGLU && rs >= 4) ? g.Wx2 : g.Wx) + (long)(grp - g.grp_x) * g.wx_gstride
                         : ((GEGLU && rs >= 4) ? g.W2 : g.W) + (long)grp * g.w_gstride;
  const bf16_t* wp = Wb + (long)min(col, g.N - 1) * (alt ? g.ldwx : g.ldw) + kb + 8 * part;
  const int nst = nk >> 6;
  const int st_lo = (kw * nst) / KW, st_hi = ((kw + 1) * nst) / KW;
  // the first batch of weight loads goes out before the activation staging
  bf16x8 w[U];
  if (st_lo < st_hi) {
#pragma unroll
    for (int j = 0; j < U; ++j) w[j] = load_bf16x8(wp + 64 * min(st_lo + j, st_hi - 1));
  }

  // stage the activation rows (16 bytes per thread and pass; rows past the
  // item's end are zero)
  const int c16 = nk >> 3;
  for (int i = tid; i < RB * c16; i += 256) {
    const int r = i / c16, c = i - r * c16;
    bf16x8 v;
    if (r < nrows) {
      const int ar = g.a_rows ? g.a_rows[r0 + r] : r0 + r;
      v = load_bf16x8(g.A + (long)ar * g.lda + kb + 8 * c);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.f;
    }
    *reinterpret_cast<bf16x8*>(&X[r * nk + 8 * c]) = v;
  }
  __syncthreads();

  const bf16_t* xp = X + 8 * part;
  float acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = 0.f;
  for (int s0 = st_lo; s0 < st_hi; s0 += U) {
    if (s0 != st_lo) {
#pragma unroll
      for (int j = 0; j < U; ++j) w[j] = load_bf16x8(wp + 64 * min(s0 + j, st_hi - 1));
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (s0 + j < st_hi) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const bf16x8 xv = *reinterpret_cast<const bf16x8*>(xp + r * nk + 64 * (s0 + j));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 wa = {w[j][2 * e], w[j][2 * e + 1]};
            const bf16x2 xa = {xv[2 * e], xv[2 * e + 1]};
            acc[r] = __builtin_amdgcn_fdot2_f32_bf16(wa, xa, acc[r], false);
          }
        }
      }
    }
  }
  // sum the 8 parts of each row (lanes 8 rs .. 8 rs + 7), then the KW waves
  // of the row set (in k order)
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    acc[r] += __shfl_xor(acc[r], 1, 64);
    acc[r] += __shfl_xor(acc[r], 2, 64);
    acc[r] += __shfl_xor(acc[r], 4, 64);
  }
  if (KW > 1) {
    if (part == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) red[wave][rs][r] = acc[r];
    }
    __syncthreads();
    if (kw != 0) return;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float v = red[wave][rs][r];
#pragma unroll
      for (int q = 1; q < KW; ++q) v += red[wave + q][rs][r];
      acc[r] = v;
    }
  }
  float up[RB];
  if (GEGLU) {
#pragma unroll
    for (int r = 0; r < RB; ++r) up[r] = __shfl(acc[r], (lane + 32) & 63, 64);
  }
  if (part != 0 || col >= g.N || (GEGLU && rs >= 4)) return;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if (r >= nrows) break;
    const float v = acc[r];
    const long off = (long)(r0 + r) * g.ldc + col;
    if (EPI == EPI_STORE_BF16) {
      reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(v);
    } else if (EPI == EPI_STORE_F32) {
      reinterpret_cast<float*>(g.C)[(long)zk * g.c_kstride + off] = v;
    } else {
      reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(gelu_tanh(v) * up[r]);
    }
  }
}

template <int EPI, bool ITEMS, int RB, int KW>
static hipError_t gemv_launch(const GemmArgs& a, hipStream_t s) {
  constexpr int NCOL = gemv_cols<KW>(EPI == EPI_GEGLU_BF16);
  const long units = (ITEMS ? (long)a.items_max : 1L) * ((a.N + NCOL - 1) / NCOL) * a.k_split;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemv_kernel<EPI, ITEMS, RB, KW>), dim3(units), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int EPI, bool ITEMS, int RB>
static hipError_t gemv_split(const GemmArgs& a, hipStream_t s) {
  const int nst = a.k_chunk / 64;   // longest k slice, in 128-byte steps
  if (nst <= 16) return gemv_launch<EPI, ITEMS, RB, 1>(a, s);
  if (nst <= 32) return gemv_launch<EPI, ITEMS, RB, 2>(a, s);
  return gemv_launch<EPI, ITEMS, RB, 4>(a, s);
}

template <int EPI, bool ITEMS>
static hipError_t gemv_rows(const GemmArgs& a, int rows, hipStream_t s) {
  if (rows == 1) return gemv_split<EPI, ITEMS, 1>(a, s);
  if (rows == 2) return gemv_split<EPI, ITEMS, 2>(a, s);
  return gemv_split<EPI, ITEMS, 4>(a, s);
}

hipError_t gemm(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.K % 64 != 0 || a.k_chunk % 64 != 0 || a.k_split < 1 || a.items_max < 1) return hipErrorInvalidValue;
  if (a.lda % 8 != 0 || a.ldw % 8 != 0) return hipErrorInvalidValue;   // 16-byte aligned rows
  const bool it = a.items != nullptr;
  const int few = it ? a.few_rows : a.M;
  const bool gemv = few >= 1 && few <= kGemvRows && a.k_chunk <= kGemvK;
  if (a.Wx && (!it || !gemv || a.ldwx % 8 != 0)) return hipErrorInvalidValue;   // alternate weights: GEMV only
  if (gemv) {
    switch (epi) {
      case EPI_STORE_BF16: return it ? gemv_rows<EPI_STORE_BF16, true>(a, few, s) : gemv_rows<EPI_STORE_BF16, false>(a, few, s);
      case EPI_STORE_F32: return it ? gemv_rows<EPI_STORE_F32, true>(a, few, s) : gemv_rows<EPI_STORE_F32, false>(a, few, s);
      case EPI_GEGLU_BF16: return it ? gemv_rows<EPI_GEGLU_BF16, true>(a, few, s) : gemv_rows<EPI_GEGLU_BF16, false>(a, few, s);
    }
    return hipErrorInvalidValue;
  }
  if (a.waves8 && !it) {
    switch (epi) {
      case EPI_STORE_BF16: return launch8<EPI_STORE_BF16>(a, s);
      case EPI_STORE_F32: return launch8<EPI_STORE_F32>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case EPI_STORE_BF16: return it ? launch<EPI_STORE_BF16, true>(a, s) : launch<EPI_STORE_BF16, false>(a, s);
    case EPI_STORE_F32: return it ? launch<EPI_STORE_F32, true>(a, s) : launch<EPI_STORE_F32, false>(a, s);
    case EPI_GEGLU_BF16: return it ? launch<EPI_GEGLU_BF16, true>(a, s) : launch<EPI_GEGLU_BF16, false>(a, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Wide variant for products whose activation side is large (the 256-row dense
// projections, the LM head and the soft-prediction embedding): a workgroup of
// 8 waves owns 256 activation rows x 128 weight rows, so every weight byte is
// streamed once per 256 rows.  Stages of 64 columns (A 32 KB + B 16 KB) go
// through a 3-deep LDS ring (144 KB: one workgroup per CU, two stages in
// flight).  Wave w multiplies weight rows 64*(w&1) .. +63 by activation rows
// 64*(w>>1) .. +63 (4 x 4 MFMA tiles).  Only plain stores: split-K slices are
// written as partial tiles and summed by the consumer.
constexpr int kFatA = 256 * 64, kFatStage = (256 + 128) * 64;

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_fat_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) bf16_t S0[kFatStage];
  __shared__ __attribute__((aligned(1024))) bf16_t S1[kFatStage];
  __shared__ __attribute__((aligned(1024))) bf16_t S2[kFatStage];
  if (g.flag && *g.flag) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = (g.N + 127) / 128;
  const long bidx = xcd_logical_block((long)g.items_max * ntiles * g.k_split);
  if (bidx < 0) return;
  const int item = (int)(bidx % g.items_max);
  const long rest = bidx / g.items_max;
  const int tile = (int)(rest % ntiles);
  const int zk = (int)(rest / ntiles);
  const int r0 = item * 256;
  const int nrows = min(256, g.M - r0);
  if (nrows <= 0) return;
  const int n_base = tile * 128;
  const int kb = zk * g.k_chunk;
  const int ke = min(g.K, kb + g.k_chunk);
  const int nst = (ke - kb) >> 6;
  if (nst <= 0) return;
  const bool wnt = g.items_max == 1;   // each weight tile is read by this workgroup only

  // DMA: wave w moves A row groups 4w..4w+3 and B row groups 2w, 2w+1 (8 rows
  // each).  Addresses = wave-uniform base (advanced per stage, kept in SGPRs)
  // + per-lane 32-bit byte offsets fixed for the whole loop.
  const int lrow = lane >> 3, lslot = lane & 7;
  const int part = lslot ^ lrow;
  int aoff[4], boff[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (4 * wave + j) * 8 + lrow;   // 0..255
    aoff[j] = (int)(((long)min(row, nrows - 1) * g.lda + part * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (2 * wave + j) * 8 + lrow;   // 0..127
    boff[j] = (int)(((long)(min(n_base + row, g.N - 1) - n_base) * g.ldw + part * 8) * 2);
  }
  const char* abase = reinterpret_cast<const char*>(g.A + (long)r0 * g.lda + kb);
  const char* bbase = reinterpret_cast<const char*>(g.W + (long)n_base * g.ldw + kb);
  const int dst_a = (4 * wave) * 512, dst_b = kFatA + (2 * wave) * 512;
#define DG_FISSUE(S, ST)                                                                                   \
  do {                                                                                                     \
    const char* ab_ = abase + ((long)(ST) << 7);                                                           \
    const char* bb_ = bbase + ((long)(ST) << 7);                                                           \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                          \
      __builtin_amdgcn_global_load_lds((const void*)(ab_ + aoff[j]), (lds_void_t*)&S[dst_a + 512 * j], 16, 0, 0); \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                          \
      DG_LDS_LOAD(bb_ + boff[j], &S[dst_b + 512 * j], kNT);                                                \
  } while (0)

  const int lr = lane & 15, lg = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  // B-operand row offsets computed once: derived inside the read macro, the
  // compiler lost track of which LDS array one of the reads targets and made
  // it wait for every DMA in flight.
  int boffr[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) boffr[n] = (64 * wn + 16 * n + lr) * 64;
  floatx4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Operand reads of the current stage are all issued before the next stage's
  // DMA (sched_barrier keeps that order): an LDS read after a DMA that the
  // compiler cannot prove disjoint would make it wait for every DMA in flight.
#define DG_FREAD(S)                                                                                        \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                                          \
    const int p_ = 4 * j + lg;                                                                             \
    _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                                        \
      const int arow = 64 * wm + 16 * m + lr;                                                              \
      af[j][m] = *reinterpret_cast<const bf16x8*>(&S[arow * 64 + ((p_ ^ (arow & 7)) << 3)]);               \
    }                                                                                                      \
    _Pragma("unroll") for (int n = 0; n < 4; ++n) {                                                        \
      bfr[j][n] = *reinterpret_cast<const bf16x8*>(&S[kFatA + boffr[n] + ((p_ ^ (lr & 7)) << 3)]);         \
    }                                                                                                      \
  }
#define DG_FMMA()                                                                                          \
  _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                            \
    _Pragma("unroll") for (int m = 0; m < 4; ++m)                                                          \
      _Pragma("unroll") for (int n = 0; n < 4; ++n) acc[m][n] = mfma16x16x32(af[j][m], bfr[j][n], acc[m][n]);
  // two stages in flight: when stage s is read, only stage s+1 (6 loads per lane) may be pending
#define DG_FITER(SI, CUR, NXT)                                                                             \
  do {                                                                                                     \
    const int s_ = (SI);                                                                                   \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(6));                                                             \
    __builtin_amdgcn_s_barrier();                                                                          \
    DG_FREAD(CUR);                                                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
    DG_FISSUE(NXT, min(s_ + 2, nst - 1));                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
    DG_FMMA();                                                                                             \
  } while (0)
  bf16x8 af[2][4], bfr[2][4];

  auto pipeline = [&](auto nt_tag) {
  constexpr bool kNT = decltype(nt_tag)::value;
  DG_FISSUE(S0, 0);
  DG_FISSUE(S1, min(1, nst - 1));
  int s = 0;
  for (; s + 3 <= nst; s += 3) {
    DG_FITER(s, S0, S2);
    DG_FITER(s + 1, S1, S0);
    DG_FITER(s + 2, S2, S1);
  }
  // every stage has been issued: the tail only drains the ring
#define DG_FTAIL(CUR)                                                                                      \
  do {                                                                                                     \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                                                             \
    __builtin_amdgcn_s_barrier();                                                                          \
    DG_FREAD(CUR);                                                                                         \
    DG_FMMA();                                                                                             \
  } while (0)
  if (s < nst) DG_FTAIL(S0);
  if (s + 1 < nst) DG_FTAIL(S1);
  };
  if (wnt) pipeline(std::true_type{});
  else pipeline(std::false_type{});
#undef DG_FTAIL
#undef DG_FISSUE
#undef DG_FREAD
#undef DG_FMMA
#undef DG_FITER

#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int col = n_base + 64 * wn + 16 * n + lr;
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 64 * wm + 16 * m + 4 * lg + i;
        if (rl >= nrows) continue;
        const long off = (long)(r0 + rl) * g.ldc + col;
        if (EPI == EPI_STORE_BF16) reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(acc[m][n][i]);
        else reinterpret_cast<float*>(g.C)[(long)zk * g.c_kstride + off] = acc[m][n][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Square variant for the widest products (LM head, soft-prediction embedding):
// 256 activation rows x 256 weight rows per workgroup of 8 waves, so every
// activation byte fetched feeds 256 weight rows (two request bytes per weight
// byte instead of three).  Stages of 64 columns (A 32 KB + B 32 KB) in a ring
// of two: stage s+1 streams while stage s is multiplied, and the DMA of stage
// s+2 reuses stage s's buffer once every wave has read it.  Wave w multiplies
// activation rows 128 (w / 4) .. +127 by weight rows 64 (w % 4) .. +63.
constexpr int kFat2A = 256 * 64, kFat2Stage = 512 * 64;

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_fat2_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) bf16_t S0[kFat2Stage];
  __shared__ __attribute__((aligned(1024))) bf16_t S1[kFat2Stage];
  if (g.flag && *g.flag) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = (g.N + 255) / 256;
  const long bidx = xcd_logical_block((long)g.items_max * ntiles * g.k_split);
  if (bidx < 0) return;
  const int item = (int)(bidx % g.items_max);
  const long rest = bidx / g.items_max;
  const int tile = (int)(rest % ntiles);
  const int zk = (int)(rest / ntiles);
  const int r0 = item * 256;
  const int nrows = min(256, g.M - r0);
  if (nrows <= 0) return;
  const int n_base = tile * 256;
  const int kb = zk * g.k_chunk;
  const int ke = min(g.K, kb + g.k_chunk);
  const int nst = (ke - kb) >> 6;
  if (nst <= 0) return;
  const bool wnt = g.items_max == 1;   // each weight tile is read by this workgroup only

  // DMA: wave w moves A row groups 4w..4w+3 and B row groups 4w..4w+3 (8 rows
  // each); wave-uniform bases advance per stage, per-lane byte offsets are fixed.
  const int lrow = lane >> 3, lslot = lane & 7;
  const int part = lslot ^ lrow;
  int aoff[4], boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (4 * wave + j) * 8 + lrow;   // 0..255
    aoff[j] = (int)(((long)min(row, nrows - 1) * g.lda + part * 8) * 2);
    boff[j] = (int)(((long)(min(n_base + row, g.N - 1) - n_base) * g.ldw + part * 8) * 2);
  }
  const char* abase = reinterpret_cast<const char*>(g.A + (long)r0 * g.lda + kb);
  const char* bbase = reinterpret_cast<const char*>(g.W + (long)n_base * g.ldw + kb);
  const int dst_a = (4 * wave) * 512, dst_b = kFat2A + (4 * wave) * 512;
#define DG_F2ISSUE(S, ST)                                                                                  \
  do {                                                                                                     \
    const char* ab_ = abase + ((long)(ST) << 7);                                                           \
    const char* bb_ = bbase + ((long)(ST) << 7);                                                           \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                          \
      __builtin_amdgcn_global_load_lds((const void*)(ab_ + aoff[j]), (lds_void_t*)&S[dst_a + 512 * j], 16, 0, 0); \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                          \
      DG_LDS_LOAD(bb_ + boff[j], &S[dst_b + 512 * j], kNT);                                                \
  } while (0)

  const int lr = lane & 15, lg = lane >> 4;
  const int wn = wave & 3, wm = wave >> 2;
  int boffr[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) boffr[n] = kFat2A + (64 * wn + 16 * n + lr) * 64;
  floatx4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  // A stage's operand reads run ahead of its MFMAs: the 12 reads of k half 0
  // are issued at once, and each activation fragment of k half 1 is read
  // into the registers of the same fragment of half 0 as soon as that
  // fragment's 4 MFMAs are issued (half 1's weight fragments at the start),
  // so only the first reads of a stage stall the MFMA chain.
  bf16x8 af[8], bf0[4], bf1[4];
#define DG_F2RA(S, J, M) \
  (*reinterpret_cast<const bf16x8*>(&S[(128 * wm + 16 * (M) + lr) * 64 + (((4 * (J) + lg) ^ (lr & 7)) << 3)]))
#define DG_F2RB(S, J, N) (*reinterpret_cast<const bf16x8*>(&S[boffr[N] + (((4 * (J) + lg) ^ (lr & 7)) << 3)]))
#define DG_F2STAGEMM(S)                                                                                    \
  do {                                                                                                     \
    _Pragma("unroll") for (int n = 0; n < 4; ++n) bf0[n] = DG_F2RB(S, 0, n);                               \
    _Pragma("unroll") for (int m = 0; m < 8; ++m) af[m] = DG_F2RA(S, 0, m);                                \
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);                                                    \
    _Pragma("unroll") for (int m = 0; m < 8; ++m) {                                                        \
      _Pragma("unroll") for (int n = 0; n < 4; ++n) acc[m][n] = mfma16x16x32(af[m], bf0[n], acc[m][n]);    \
      if (m == 0) {                                                                                        \
        _Pragma("unroll") for (int n = 0; n < 4; ++n) bf1[n] = DG_F2RB(S, 1, n);                           \
      }                                                                                                    \
      af[m] = DG_F2RA(S, 1, m);                                                                            \
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                                                   \
      if (m == 0) __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);                                       \
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                              \
    }                                                                                                      \
    _Pragma("unroll") for (int m = 0; m < 8; ++m)                                                          \
      _Pragma("unroll") for (int n = 0; n < 4; ++n) acc[m][n] = mfma16x16x32(af[m], bf1[n], acc[m][n]);    \
  } while (0)
  // stage s is read when at most stage s+1 (8 loads per lane) is pending; its
  // buffer is refilled (stage s+2, clamped to the last stage, so every
  // iteration issues the same count) after every wave has read it
#define DG_F2ITER(SI, CUR)                                                                                 \
  do {                                                                                                     \
    const int s_ = (SI);                                                                                   \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));                                                             \
    __builtin_amdgcn_s_barrier();                                                                          \
    DG_F2STAGEMM(CUR);                                                                                     \
    __builtin_amdgcn_s_waitcnt(0xC07F);   /* lgkmcnt(0): this wave's reads of CUR are done */              \
    __builtin_amdgcn_s_barrier();                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
    DG_F2ISSUE(CUR, min(s_ + 2, nst - 1));                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
  } while (0)

  auto pipeline = [&](auto nt_tag) {
  constexpr bool kNT = decltype(nt_tag)::value;
  DG_F2ISSUE(S0, 0);
  DG_F2ISSUE(S1, min(1, nst - 1));
  int s = 0;
  for (; s + 2 <= nst; s += 2) {
    DG_F2ITER(s, S0);
    DG_F2ITER(s + 1, S1);
  }
  if (s < nst) {   // odd count: the last stage sits in S0; drain the ring
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    DG_F2STAGEMM(S0);
  }
  };
  if (wnt) pipeline(std::true_type{});
  else pipeline(std::false_type{});
  __builtin_amdgcn_s_waitcnt(0);   // no DMA into LDS outlives the loop
#undef DG_F2ISSUE
#undef DG_F2RA
#undef DG_F2RB
#undef DG_F2STAGEMM
#undef DG_F2ITER

#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int col = n_base + 64 * wn + 16 * n + lr;
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 128 * wm + 16 * m + 4 * lg + i;
        if (rl >= nrows) continue;
        const long off = (long)(r0 + rl) * g.ldc + col;
        if (EPI == EPI_STORE_BF16) reinterpret_cast<bf16_t*>(g.C)[off] = f2bf(acc[m][n][i]);
        else reinterpret_cast<float*>(g.C)[(long)zk * g.c_kstride + off] = acc[m][n][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// C [M][N] (fp32; k slice zk at C + zk c_kstride) = A [M][K] W [K][N], the weight
// stored K-major (rows of N contiguous values): the soft-prediction product
// reads the tied embedding E [vocab][d] as stored, contracting over the
// vocabulary, so no transposed copy of E is needed.  Square 256 x 256 tiles
// and waves as gemm_fat2_kernel; the weight part of a stage is 64 rows of W
// (k) x 256 columns (n), 512 bytes per row, whose 16-byte slots are XOR-
// swizzled by 2 (k % 4) + 8 ((k / 8) % 2).  The MFMA B operand (8 consecutive k of one column
// per lane) comes from two transposed LDS reads (ds_read_b64_tr_b16): within
// each 16 lanes, lane 4a + b receives element b of the 8-byte reads of lanes
// a, a + 4, a + 8, a + 12, so lane 4a + j of 16-lane group G reads row
// 8 G + j (then 8 G + 4 + j) at column 4 a of the fragment's 16: lane t ends
// up with column t and rows 8 G .. 8 G + 7, the k-slots of the A operand's
// 16-byte reads.  The eight rows that 32 lanes read (k % 4 and k / 8 vary)
// sit in eight distinct slot pairs of a 256-byte bank row, so the reads are
// bank-conflict-free.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ int kn_swz(int row) { return 2 * (row & 3) + 8 * ((row >> 3) & 1); }

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_kn_kernel(GemmArgs g) {
  static_assert(EPI == EPI_STORE_F32, "split-K partials");
  __shared__ __attribute__((aligned(1024))) bf16_t S0[kFat2Stage];
  __shared__ __attribute__((aligned(1024))) bf16_t S1[kFat2Stage];
  if (g.flag && *g.flag) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = (g.N + 255) / 256;
  const long bidx = xcd_logical_block((long)g.items_max * ntiles * g.k_split);
  if (bidx < 0) return;
  const int item = (int)(bidx % g.items_max);
  const long rest = bidx / g.items_max;
  const int tile = (int)(rest % ntiles);
  const int zk = (int)(rest / ntiles);
  const int r0 = item * 256;
  const int nrows = min(256, g.M - r0);
  if (nrows <= 0) return;
  const int n_base = tile * 256;
  const int kb = zk * g.k_chunk;
  const int ke = min(g.K, kb + g.k_chunk);
  const int nst = (ke - kb) >> 6;
  if (nst <= 0) return;
  const bool wnt = g.items_max == 1;   // each weight tile is read by this workgroup only

  // DMA.  A: wave w moves row groups 4w..4w+3 (8 rows of 128 B each, as
  // gemm_fat2_kernel).  W: wave w moves W rows 8w .. 8w + 7, two per
  // instruction (lane l: row + l / 32, LDS slot l % 32 holding global part
  // (l % 32) ^ kn_swz(row), clamped to the last 16 bytes of the row); a stage
  // advances 64 rows of W.
  const int lrow = lane >> 3, lslot = lane & 7;
  const int part = lslot ^ lrow;
  int aoff[4], boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (4 * wave + j) * 8 + lrow;   // 0..255
    aoff[j] = (int)(((long)min(row, nrows - 1) * g.lda + part * 8) * 2);
    const int wr = 8 * wave + 2 * j + (lane >> 5);   // 0..63
    const int col = min(n_base + 8 * ((lane & 31) ^ kn_swz(wr)), g.N - 8);
    boff[j] = (int)(((long)wr * g.ldw + col) * 2);
  }
  const char* abase = reinterpret_cast<const char*>(g.A + (long)r0 * g.lda + kb);
  const char* bbase = reinterpret_cast<const char*>(g.W + (long)kb * g.ldw);
  const long bstep = (long)64 * g.ldw * 2;   // bytes per stage of W rows
  const int dst_a = (4 * wave) * 512, dst_b = kFat2A + (8 * wave) * 256;
#define DG_KNISSUE(S, ST)                                                                                  \
  do {                                                                                                     \
    const char* ab_ = abase + ((long)(ST) << 7);                                                           \
    const char* bb_ = bbase + (long)(ST) * bstep;                                                          \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                          \
      __builtin_amdgcn_global_load_lds((const void*)(ab_ + aoff[j]), (lds_void_t*)&S[dst_a + 512 * j], 16, 0, 0); \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                          \
      DG_LDS_LOAD(bb_ + boff[j], &S[dst_b + 512 * j], kNT);                                                \
  } while (0)

  const int lr = lane & 15, lg = lane >> 4;
  const int wn = wave & 3, wm = wave >> 2;
  // transposed B reads: lane 4 a + jr of group lg reads row 8 lg + jr (+ 4) at column 4 a
  const int ta = lr & 3, tj = lr >> 2;
  int bcol[4];   // element offset of this lane's 8-byte read within a W row, per 16-column block
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int c = 64 * wn + 16 * n + 4 * ta;
    bcol[n] = c;   // part c / 8, half (c % 8) / 4
  }
  floatx4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  // operand reads run ahead of the MFMAs as in gemm_fat2_kernel
  bf16x8 af[8], bf0[4], bf1[4];
#define DG_KNB(S, ROW, C)                                                                                  \
  __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                                                 \
      (lds_v4i16_t*)&S[kFat2A + (ROW) * 256 + ((((C) >> 3) ^ kn_swz(ROW)) << 3) + ((C) & 4)])
#define DG_KNRA(S, J, M) \
  (*reinterpret_cast<const bf16x8*>(&S[(128 * wm + 16 * (M) + lr) * 64 + (((4 * (J) + lg) ^ (lr & 7)) << 3)]))
#define DG_KNRB(S, J, DST)                                                                                 \
  do {                                                                                                     \
    const int r0_ = 32 * (J) + 8 * lg + tj;                                                                \
    _Pragma("unroll") for (int n = 0; n < 4; ++n) {                                                        \
      const v4i16_t lo_ = DG_KNB(S, r0_, bcol[n]);                                                         \
      const v4i16_t hi_ = DG_KNB(S, r0_ + 4, bcol[n]);                                                     \
      const v8i16_t both_ = __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3, 4, 5, 6, 7);                    \
      DST[n] = __builtin_bit_cast(bf16x8, both_);                                                          \
    }                                                                                                      \
  } while (0)
#define DG_KNSTAGEMM(S)                                                                                    \
  do {                                                                                                     \
    DG_KNRB(S, 0, bf0);                                                                                    \
    _Pragma("unroll") for (int m = 0; m < 8; ++m) af[m] = DG_KNRA(S, 0, m);                                \
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);                                                    \
    _Pragma("unroll") for (int m = 0; m < 8; ++m) {                                                        \
      _Pragma("unroll") for (int n = 0; n < 4; ++n) acc[m][n] = mfma16x16x32(af[m], bf0[n], acc[m][n]);    \
      if (m == 0) DG_KNRB(S, 1, bf1);                                                                      \
      af[m] = DG_KNRA(S, 1, m);                                                                            \
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                                                   \
      if (m == 0) __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);                                       \
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                              \
    }                                                                                                      \
    _Pragma("unroll") for (int m = 0; m < 8; ++m)                                                          \
      _Pragma("unroll") for (int n = 0; n < 4; ++n) acc[m][n] = mfma16x16x32(af[m], bf1[n], acc[m][n]);    \
  } while (0)
#define DG_KNITER(SI, CUR)                                                                                 \
  do {                                                                                                     \
    const int s_ = (SI);                                                                                   \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));                                                             \
    __builtin_amdgcn_s_barrier();                                                                          \
    DG_KNSTAGEMM(CUR);                                                                                     \
    __builtin_amdgcn_s_waitcnt(0xC07F);   /* lgkmcnt(0): this wave's reads of CUR are done */              \
    __builtin_amdgcn_s_barrier();                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
    DG_KNISSUE(CUR, min(s_ + 2, nst - 1));                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                                     \
  } while (0)

  auto pipeline = [&](auto nt_tag) {
    constexpr bool kNT = decltype(nt_tag)::value;
    DG_KNISSUE(S0, 0);
    DG_KNISSUE(S1, min(1, nst - 1));
    int s = 0;
    for (; s + 2 <= nst; s += 2) {
      DG_KNITER(s, S0);
      DG_KNITER(s + 1, S1);
    }
    if (s < nst) {   // odd count: the last stage sits in S0; drain the ring
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_barrier();
      DG_KNSTAGEMM(S0);
    }
  };
  if (wnt) pipeline(std::true_type{});
  else pipeline(std::false_type{});
  __builtin_amdgcn_s_waitcnt(0);   // no DMA into LDS outlives the loop
#undef DG_KNISSUE
#undef DG_KNB
#undef DG_KNRA
#undef DG_KNRB
#undef DG_KNSTAGEMM
#undef DG_KNITER

#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int col = n_base + 64 * wn + 16 * n + lr;
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 128 * wm + 16 * m + 4 * lg + i;
        if (rl >= nrows) continue;
        const long off = (long)(r0 + rl) * g.ldc + col;
        reinterpret_cast<float*>(g.C)[(long)zk * g.c_kstride + off] = acc[m][n][i];
      }
    }
  }
}

hipError_t gemm_kn(const GemmArgs& a, hipStream_t s) {
  if (a.K % 64 != 0 || a.k_chunk % 64 != 0 || a.k_split < 1 || a.items_max < 1) return hipErrorInvalidValue;
  if (a.lda % 8 != 0 || a.ldw % 8 != 0 || a.N % 8 != 0 || a.N < 8 || a.items || a.a_rows) return hipErrorInvalidValue;
  // 32-bit per-lane offsets: 256 rows of A, 64 rows of W
  if (256L * a.lda * 2 >= 0x7FFFFFFFL || (64L * a.ldw + a.N) * 2 >= 0x7FFFFFFFL) return hipErrorInvalidValue;
  const long total = (long)a.items_max * ((a.N + 255) / 256) * a.k_split;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_kn_kernel<EPI_STORE_F32>, dim3(xcd_grid(total)), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t gemm_fat2(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.K % 64 != 0 || a.k_chunk % 64 != 0 || a.k_split < 1 || a.items_max < 1) return hipErrorInvalidValue;
  if (a.lda % 8 != 0 || a.ldw % 8 != 0 || a.items || a.a_rows) return hipErrorInvalidValue;
  if (!gemm_fat2_pitch_ok(a.lda, a.ldw)) return hipErrorInvalidValue;   // 32-bit per-lane offsets
  const long total = (long)a.items_max * ((a.N + 255) / 256) * a.k_split;
  if (total <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE_F32: hipLaunchKernelGGL(gemm_fat2_kernel<EPI_STORE_F32>, dim3(xcd_grid(total)), dim3(512), 0, s, a); break;
    case EPI_STORE_BF16: hipLaunchKernelGGL(gemm_fat2_kernel<EPI_STORE_BF16>, dim3(xcd_grid(total)), dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t gemm_fat(int epi, const GemmArgs& a, hipStream_t s) {
  if (a.K % 64 != 0 || a.k_chunk % 64 != 0 || a.k_split < 1 || a.items_max < 1) return hipErrorInvalidValue;
  if (a.lda % 8 != 0 || a.ldw % 8 != 0 || a.items || a.a_rows) return hipErrorInvalidValue;
  if (!gemm_fat_pitch_ok(a.lda, a.ldw)) return hipErrorInvalidValue;   // 32-bit per-lane offsets
  const long total = (long)a.items_max * ((a.N + 127) / 128) * a.k_split;
  if (total <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE_F32: hipLaunchKernelGGL(gemm_fat_kernel<EPI_STORE_F32>, dim3(xcd_grid(total)), dim3(512), 0, s, a); break;
    case EPI_STORE_BF16: hipLaunchKernelGGL(gemm_fat_kernel<EPI_STORE_BF16>, dim3(xcd_grid(total)), dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dg
