// Canvas / prefix attention on MFMA for gfx950, flash-style with key splits.
//
// Mask (DiffusionGemma: causal prompt encoding, bidirectional canvas; laozijiushiniubi
// article section 2, gxsgwd news item): canvas queries see every prefix key and
// every canvas key of their own canvas; prefix queries (prefill) see keys at
// positions <= their own.  Query head h reads key/value head h / (H / Hkv).
//
// Work split.  A workgroup of NW waves owns 16 NW NF (query, head) rows that
// share one key/value head: 16 NW NF / GQ queries times the GQ query heads of
// that kv head, as NW NF row fragments of 16.  Each wave holds NF fragments, so
// every key / value fragment it reads from LDS feeds NF MFMAs (shapes per
// head_dim: attn_waves / attn_frags).  Workgroups also split the keys; a merge
// combines the splits.
//
// Key / value tiles (32 keys) stream through a 4-deep LDS ring by direct
// global->LDS DMA: K rows [32][hd] and V^T rows [hd][32 keys] (the V^T caches
// are stored tile-major, so a tile's V^T is one contiguous block), 16-byte slots
// XOR-swizzled (K: slot ^ kswz(key), V^T: slot ^ vswz(dim)) so that the 16
// lanes that one LDS pass of a 16-byte read serves hit distinct banks.  The
// V^T swizzle was chosen by measurement (a bank-conflict counter probe of all
// 256 linear swizzles of the row's low 4 bits over the 16 rows of 64 bytes
// that a pass reads: 96 read conflict-free, the rest 2- or 4-way).
//
// Each fragment computes S^T = K Q^T with keys as the MFMA M dimension.  The
// K fragment of block kf reads key row 8 (r / 4) + 4 kf + r % 4 for MFMA row
// r, so a lane ends up with the 8 consecutive keys 8 (l / 16) .. + 7 of ONE
// query row: as bf16 probabilities they are the A operand of P V, and the B
// operand is one 16-byte read of a V^T row.  Scores are scaled to log2 units
// inside the exponent.  The running max is raised lazily: the accumulator is
// rescaled only when a row's max grows by more than 8 (probabilities then stay
// below 2^8), which happens on the first tiles and rarely after.  Only tiles
// that cross the causal diagonal or the end of the keys are masked.  Each lane
// keeps a partial row sum of its own keys; the four partials of a row are
// added once at the end.  Outputs: the normalised O of each split in bf16
// plus (max, sum) per row, or the final O when there is one split.
#include <math.h>

#include "dg_kernels.hpp"

namespace dg {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int waitcnt_vm_attn(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// slot swizzles: K row `key` (0..31 in the tile) of a head_dim with ck 16-byte
// slots, and V^T row `dim`
__device__ __forceinline__ int kswz(int key, int ck) { return ((key & 3) | ((key >> 1) & 12)) & (ck - 1); }
__device__ __forceinline__ int vswz(int dim) { return (dim >> 1) & 3; }

// sum / max over the four lanes l % 16 + 16 i of a wave (gfx950 row swaps)
__device__ __forceinline__ float xrow_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float xrow_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int HD, int GQ, int NW, int NF>
__global__ __launch_bounds__(64 * NW, 1) void attn_kernel(AttnArgs a) {
  constexpr int APD = HD / 16 < 8 ? HD / 16 : 8;   // V^T blocks read ahead of the P V MFMAs
  constexpr int KS = HD / 32;          // 32-wide contraction steps of S over hd
  constexpr int NFD = HD / 16;         // 16-wide blocks of O over hd
  constexpr int CK = HD / 8;           // 16-byte slots per K row
  constexpr int KSB = KS < 4 ? KS : 4;  // distinct K read offsets per block (swizzle period 16 slots)
  constexpr int SE = 64 * HD;          // stage: K [32][HD] then V^T [HD][32], bf16 elements
  constexpr int IPW = HD / 8 / NW;     // 1 KB DMA instructions per wave per stage
  constexpr int KI = HD / 16 / NW;     // of which the first KI move K rows
  static_assert(KI >= 1 && IPW == 2 * KI, "K and V^T tiles split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) bf16_t S0[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S1[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S2[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S3[SE];
  if (a.flag && *a.flag) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int QPW = 16 * NW * NF / GQ;   // queries per workgroup
  const int R = a.rows_per_batch;
  const int nqb = (R + QPW - 1) / QPW;
  // query blocks fastest: the blocks that read one (kv head, key split) share an XCD
  const long lb = xcd_logical_block((long)nqb * a.Hkv * a.splits * a.B);
  if (lb < 0) return;
  const int qb = (int)(lb % nqb);
  const int gy = (int)((lb / nqb) % (a.Hkv * a.splits));
  const int b = (int)(lb / ((long)nqb * a.Hkv * a.splits));
  const int g = gy % a.Hkv, split = gy / a.Hkv;
  const int q0wg = qb * QPW;
  const int lr = lane & 15, lg = lane >> 4;

  const int qpos0 = a.pos_dev ? *a.pos_dev : a.qpos0;
  const int n1 = a.pos_dev ? (qpos0 + R + 31) & ~31 : a.n1;
  const int nk = n1 + a.n2;
  const int kbeg = split * a.split_len;
  int kend = min(nk, kbeg + a.split_len);
  if (a.causal) kend = min(kend, qpos0 + min(q0wg + QPW, R));
  const int ntile = kend > kbeg ? (kend - kbeg + 31) / 32 : 0;

  const int b1 = (a.nb1 == 1) ? 0 : b;
  const bf16_t* K1 = a.k1 + b1 * a.k1_bstride + g * a.k1_hstride;
  const bf16_t* V1 = a.vt1 + b1 * a.v1_bstride + g * a.v1_hstride;
  const bf16_t* K2 = a.k2 ? a.k2 + b * a.k2_bstride + g * a.k2_hstride : K1;
  const bf16_t* V2 = a.vt2 ? a.vt2 + b * a.v2_bstride + g * a.v2_hstride : V1;

  // ---- fragments of this wave: f = 4 wave + j -> head g*GQ + f%GQ, queries q0wg + 16 (f/GQ) + lr
  bf16x8 qfr[NF][KS];
  const bf16_t* qptr[NF];
  int qrow[NF], qpos[NF];
  bool live[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int f = NF * wave + j;
    const int h = g * GQ + f % GQ;
    const int qr0 = q0wg + 16 * (f / GQ);
    live[j] = qr0 < R;
    qrow[j] = qr0;
    const int myq = min(qr0 + lr, R - 1);
    qpos[j] = qpos0 + myq;
    qptr[j] = a.q + ((long)(b * R + myq) * a.H + h) * HD + lg * 8;
  }

  // ---- DMA sources: every key count is a multiple of 32, so a tile lies in one
  // source; per-lane element offsets within a tile are fixed for the whole loop
  int soff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    if (j < KI) {
      constexpr int KPI = 512 / HD;                     // keys per instruction
      const int key = (wave + NW * j) * KPI + lane / CK;
      const int c = (lane % CK) ^ kswz(key, CK);
      soff[j] = key * HD + c * 8;
    } else {
      // a V^T tile is a contiguous [HD][32] block: one instruction moves 16 whole rows (1 KB)
      const int row = (wave + NW * (j - KI)) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ vswz(row);
      soff[j] = row * 32 + c * 8;
    }
  }
#define DG_AISSUE(S, KT)                                                                           \
  do {                                                                                             \
    const int kt_ = (KT);                                                                          \
    const bool one_ = kt_ < n1;                                                                    \
    const bf16_t* kb_ = one_ ? K1 + (long)kt_ * HD : K2 + (long)(kt_ - n1) * HD;                   \
    const bf16_t* vb_ = one_ ? V1 + (long)(kt_ >> 5) * (32 * HD) : V2 + (long)((kt_ - n1) >> 5) * (32 * HD); \
    _Pragma("unroll") for (int j = 0; j < IPW; ++j) {                                              \
      const bf16_t* src_ = (j < KI ? kb_ : vb_) + soff[j];                                         \
      const int dst_ = (j < KI ? (wave + NW * j) : 32 * HD / 512 + (wave + NW * (j - KI))) * 512;  \
      __builtin_amdgcn_global_load_lds((const void*)src_, (lds_void_t*)&S[dst_], 16, 0, 0);        \
    }                                                                                              \
  } while (0)

  // LDS read offsets.  K block kf, step ks: key row kr = 8 (lr / 4) + 4 kf +
  // lr % 4, global slot 4 ks + lg at LDS slot (4 ks + lg) ^ kswz(kr), i.e.
  // koff[kf][ks % 4] + 128 (ks / 4) elements.  V^T block nf: row 16 nf + lr,
  // slot lg, i.e. voff[nf % 2] + 512 nf.
  int koff[2][KSB];
#pragma unroll
  for (int kf = 0; kf < 2; ++kf) {
    const int kr = 8 * (lr >> 2) + 4 * kf + (lr & 3);
#pragma unroll
    for (int q = 0; q < KSB; ++q) koff[kf][q] = kr * HD + (((4 * q + lg) ^ kswz(kr, CK)) << 3);
  }
  int voff[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) voff[e] = 32 * HD + lr * 32 + ((lg ^ vswz(16 * e + lr)) << 3);

  floatx4 O[NF][NFD];
#pragma unroll
  for (int j = 0; j < NF; ++j)
#pragma unroll
    for (int nf = 0; nf < NFD; ++nf) O[j][nf] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run[NF], l_run[NF];   // l_run: this lane's partial sum until the end
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }
  const float sl2 = a.scale * 1.4426950408889634f;
  // keys below this bound are visible to every query of the workgroup
  const int kfull = a.causal ? min(kend, qpos0 + q0wg + 1) : kend;

// Raw scores S^T = K Q^T of the tile in stage S, into SC (two chains of MFMAs
// interleaved over the head dim)
#define DG_ASCORE(S, SC)                                                                           \
  do {                                                                                             \
    _Pragma("unroll") for (int j = 0; j < NF; ++j) SC[j][0] = SC[j][1] = floatx4{0.f, 0.f, 0.f, 0.f}; \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks)                                              \
      _Pragma("unroll") for (int kf = 0; kf < 2; ++kf) {                                           \
        const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(&S[koff[kf][ks % KSB] + 128 * (ks / KSB)]); \
        _Pragma("unroll") for (int j = 0; j < NF; ++j)                                             \
          SC[j][kf] = mfma16x16x32(kfr, qfr[j][ks], SC[j][kf]);                                    \
      }                                                                                            \
  } while (0)

// -inf for the keys of tile KT that a query may not see
#define DG_AMASK(SC, KT)                                                                           \
  do {                                                                                             \
    _Pragma("unroll") for (int j = 0; j < NF; ++j)                                                 \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                              \
        const int key = (KT) + 8 * lg + e;                                                         \
        if (!(key < kend && (!a.causal || key <= qpos[j]))) SC[j][e >> 2][e & 3] = -INFINITY;      \
      }                                                                                            \
  } while (0)

// Probabilities of the scores SC against the running max, as bf16 in PF; the
// row sums go to l_run.  The exponentials are taken first against the current
// max; a row whose max grew by more than 8 (log2 units) raises it, rescales its
// accumulator and takes them again (the first tiles, rarely after).  A row
// with no visible key yet (max -inf) gets zeros.
#define DG_ASOFT(SC, PF)                                                                           \
  do {                                                                                             \
    float mx_[NF], ps_[NF];                                                                        \
    bool up_ = false;                                                                              \
    _Pragma("unroll") for (int j = 0; j < NF; ++j) {                                               \
      float p[8];                                                                                  \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) p[e] = SC[j][e >> 2][e & 3];                   \
      float mx = fmaxf(fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3])), fmaxf(fmaxf(p[4], p[5]), fmaxf(p[6], p[7]))); \
      mx = xrow_max(mx) * sl2;                                                                     \
      mx_[j] = mx;                                                                                 \
      up_ = up_ || (mx > m_run[j] + 8.0f);                                                         \
      const float nm = m_run[j] == -INFINITY ? 0.f : -m_run[j];                                    \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(p[e], sl2, nm)); \
      ps_[j] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));                 \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) PF[j][e] = (__bf16)p[e];                       \
      /* keeps this path ahead of the branch, beside the MFMAs (not sunk into its else) */         \
      asm volatile("" ::"v"(PF[j]), "v"(ps_[j]));                                                  \
    }                                                                                              \
    if (__builtin_amdgcn_ballot_w64(up_)) {                                                        \
      _Pragma("unroll") for (int j = 0; j < NF; ++j) {                                             \
        const float m_new = fmaxf(m_run[j], mx_[j]);                                               \
        const float alpha = (m_run[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[j] - m_new); \
        l_run[j] *= alpha;                                                                         \
        m_run[j] = m_new;                                                                          \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                            \
          const float ai = __shfl(alpha, lg * 4 + i, 64);                                          \
          _Pragma("unroll") for (int nf = 0; nf < NFD; ++nf) O[j][nf][i] *= ai;                    \
        }                                                                                          \
        const float nm = m_new == -INFINITY ? 0.f : -m_new;                                        \
        float p[8];                                                                                \
        _Pragma("unroll") for (int e = 0; e < 8; ++e)                                              \
          p[e] = __builtin_amdgcn_exp2f(fmaf(SC[j][e >> 2][e & 3], sl2, nm));                      \
        ps_[j] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));               \
        _Pragma("unroll") for (int e = 0; e < 8; ++e) PF[j][e] = (__bf16)p[e];                     \
      }                                                                                            \
    }                                                                                              \
    _Pragma("unroll") for (int j = 0; j < NF; ++j) l_run[j] += ps_[j];                             \
  } while (0)

// O += P V with V^T of the tile in stage S.  The reads run APD blocks ahead of
// the MFMAs (sched_group_barrier keeps that order): the compiler otherwise read
// two V^T blocks, waited for them, and issued their MFMAs, exposing an LDS
// round trip every two MFMAs
#define DG_APV(S, PF)                                                                              \
  do {                                                                                             \
    bf16x8 vb_[NFD];                                                                               \
    _Pragma("unroll") for (int nf = 0; nf < NFD; ++nf)                                             \
      vb_[nf] = *reinterpret_cast<const bf16x8*>(&S[voff[nf & 1] + 512 * nf]);                     \
    _Pragma("unroll") for (int nf = 0; nf < NFD; ++nf)                                             \
      _Pragma("unroll") for (int j = 0; j < NF; ++j) O[j][nf] = mfma16x16x32(PF[j], vb_[nf], O[j][nf]); \
    __builtin_amdgcn_sched_group_barrier(0x100, APD, 0);                                           \
    _Pragma("unroll") for (int nf = 0; nf < NFD; ++nf) {                                           \
      __builtin_amdgcn_sched_group_barrier(0x008, NF, 0);                                          \
      if (nf + APD < NFD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                       \
    }                                                                                              \
  } while (0)

  // Software pipeline over a ring of 4 stages.  Iteration T holds the scores
  // of tile T in SCUR; it waits for tile T+1 (tile T+2 may still be in
  // flight), computes the scores of tile T+1 into SNXT from stage KB while the
  // softmax of tile T runs, then P V from stage VB.  The scores of the tile
  // past the last are computed from a clamped copy and dropped.  The DMA of
  // tile T+3 (clamped to the last tile, so every iteration issues the same
  // count) follows every LDS read of the iteration and goes to the stage of
  // tile T-1, which every wave left before this iteration's barrier.
#define DG_AITER(T, VB, KB, DB, SCUR, SNXT)                                                        \
  do {                                                                                             \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_attn(IPW));                                              \
    __builtin_amdgcn_s_barrier();                                                                  \
    const int kt_ = kbeg + 32 * (T);                                                               \
    if (kt_ + 32 > kfull) DG_AMASK(SCUR, kt_);                                                     \
    bf16x8 pf_[NF];                                                                                \
    DG_ASCORE(KB, SNXT);                                                                           \
    DG_ASOFT(SCUR, pf_);                                                                           \
    DG_APV(VB, pf_);                                                                               \
    __builtin_amdgcn_sched_barrier(0);                                                             \
    DG_AISSUE(DB, kbeg + 32 * min((T) + 3, ntile - 1));                                            \
    __builtin_amdgcn_sched_barrier(0);                                                             \
  } while (0)

  if (ntile > 0) {
    // the Q fragments load ahead of the first three tiles; they retire first,
    // so waiting for them leaves the tiles in flight
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qfr[j][ks] = load_bf16x8(qptr[j] + 32 * ks);
    __builtin_amdgcn_sched_barrier(0);
    DG_AISSUE(S0, kbeg);
    DG_AISSUE(S1, kbeg + 32 * min(1, ntile - 1));
    DG_AISSUE(S2, kbeg + 32 * min(2, ntile - 1));
    floatx4 sa[NF][2], sb[NF][2];
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_attn(2 * IPW));
    __builtin_amdgcn_s_barrier();
    DG_ASCORE(S0, sa);
    // full rounds of four, then the last 0-3 tiles: a loop without early
    // exits keeps the compiler from draining the ring at its head
    int t = 0;
    for (; t + 4 <= ntile; t += 4) {
      DG_AITER(t, S0, S1, S3, sa, sb);
      DG_AITER(t + 1, S1, S2, S0, sb, sa);
      DG_AITER(t + 2, S2, S3, S1, sa, sb);
      DG_AITER(t + 3, S3, S0, S2, sb, sa);
    }
    if (t < ntile) DG_AITER(t, S0, S1, S3, sa, sb);
    if (t + 1 < ntile) DG_AITER(t + 1, S1, S2, S0, sb, sa);
    if (t + 2 < ntile) DG_AITER(t + 2, S2, S3, S1, sa, sb);
  }
#undef DG_AITER
#undef DG_APV
#undef DG_ASOFT
#undef DG_AMASK
#undef DG_ASCORE
#undef DG_AISSUE
  __builtin_amdgcn_s_waitcnt(0);

  // ---- outputs: normalised O (bf16) of this split, and (max, sum) per row
  const long BR = (long)a.B * R;
#pragma unroll
  for (int j = 0; j < NF; ++j) l_run[j] = xrow_sum(l_run[j]);
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    if (!live[j]) continue;
    const int h = g * GQ + (NF * wave + j) % GQ;
    const float inv = l_run[j] > 0.f ? 1.0f / l_run[j] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = qrow[j] + lg * 4 + i;
      const float iv = __shfl(inv, lg * 4 + i, 64);
      if (row >= R) continue;
      bf16_t* op = (a.splits == 1 ? a.out + ((long)b * R + row) * a.H * HD
                                  : a.opart + (((long)split * BR + (long)b * R + row) * a.H) * HD) + (long)h * HD;
#pragma unroll
      for (int nf = 0; nf < NFD; ++nf) op[nf * 16 + lr] = f2bf(O[j][nf][i] * iv);
    }
    if (a.splits > 1 && lg == 0 && qrow[j] + lr < R) {
      float* mp = a.mlpart + (((long)split * BR + (long)b * R + qrow[j] + lr) * a.H + h) * 2;
      mp[0] = m_run[j];
      mp[1] = l_run[j];
    }
  }
}

template <int HD, int GQ, int NW, int NF>
static void attn_launch(const AttnArgs& a, hipStream_t s) {
  const long total = (long)((a.rows_per_batch + 16 * NW * NF / GQ - 1) / (16 * NW * NF / GQ)) * a.Hkv * a.splits * a.B;
  if (total <= 0) return;
  hipLaunchKernelGGL((attn_kernel<HD, GQ, NW, NF>), dim3(xcd_grid(total)), dim3(64 * NW), 0, s, a);
}

// Workgroup shapes (waves x fragments per wave), measured on the 2816-wide
// model: at head_dim 256 eight waves of one fragment (two waves per SIMD, so
// one wave's softmax overlaps the other's MFMAs) beat four waves of two, whose
// halved LDS traffic does not pay for the lost overlap; smaller heads fit
// four fragments per wave.
template <int HD, int GQ>
static void attn_shape(const AttnArgs& a, hipStream_t s) {
  constexpr int NW = attn_waves(HD), NF = attn_frags(HD);
  attn_launch<HD, GQ, NW, NF>(a, s);
}

// ---------------------------------------------------------------------------
// Decoding: at most 8 (query, head) rows per kv head (one token, or a few, per
// sequence) over a causal prefix.  The 16-row MFMA tile and its LDS ring would
// move every K/V tile for 1-2 live rows, so a workgroup of 8 waves takes one
// (sequence, kv head, key split) and issues all its K and V^T loads at once
// (one round trip), straight to registers:
//   scores: LPK = HD / 32 lanes per key, each with 32 dims of the K row (four
//           16-byte loads) against the NQ query rows held in LDS, summed over
//           the LPK lanes by shuffles (bf16 pair products in fp32, dot2);
//   softmax: wave q takes query row q over the split's keys in LDS (max in
//           log2 units, exp2, sum), as the MFMA kernel's (m, l);
//   P V:    8 lanes per V^T row read 64 consecutive keys (two 64-byte runs of
//           the tile-major cache), summed over the 8 lanes.
// Outputs match the MFMA kernel's: normalised O per split plus (m, l), merged
// by attention_merge, or the final O for one split.
constexpr int kDecThreads = 512;
constexpr int dec_max_keys(int hd) { return 4 * kDecThreads / (hd / 32); }   // 4 passes of keys

template <int HD, int NQ>
__global__ __launch_bounds__(kDecThreads) void attn_decode_kernel(AttnArgs a) {
  constexpr int LPK = HD / 32;              // lanes per key
  constexpr int KPP = kDecThreads / LPK;    // keys per pass
  constexpr int MAXK = 4 * KPP;             // keys per split
  constexpr int VCH = MAXK / 64;            // 64-key chunks of a V^T row
  constexpr int VDP = HD / 64;              // dim passes of P V (64 rows each)
  __shared__ __attribute__((aligned(16))) bf16_t Qs[NQ * HD];
  __shared__ __attribute__((aligned(16))) float Ps[NQ * MAXK];
  if (a.flag && *a.flag) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int GQ = a.H / a.Hkv, R = a.rows_per_batch, nq = R * GQ;
  const int split = blockIdx.x % a.splits;
  const int g = (blockIdx.x / a.splits) % a.Hkv;
  const int b = blockIdx.x / (a.splits * a.Hkv);
  const int qpos0 = a.pos_dev ? *a.pos_dev : a.qpos0;
  const int n1 = a.pos_dev ? (qpos0 + R + 31) & ~31 : a.n1;
  const int kbeg = split * a.split_len;
  const int kend = min(min(n1, kbeg + a.split_len), qpos0 + R);   // causal: keys up to the last row
  const int b1 = (a.nb1 == 1) ? 0 : b;
  const bf16_t* K1 = a.k1 + b1 * a.k1_bstride + g * a.k1_hstride;
  const bf16_t* V1 = a.vt1 + b1 * a.v1_bstride + g * a.v1_hstride;

  // all K and V^T loads first
  const int kpart = tid % LPK, kslot = tid / LPK;
  bf16x8 kv[4][4];
#pragma unroll
  for (int ps = 0; ps < 4; ++ps) {
    const int key = kbeg + ps * KPP + kslot;
    if (key < kend) {
#pragma unroll
      for (int i = 0; i < 4; ++i) kv[ps][i] = load_bf16x8(K1 + (long)key * HD + 32 * kpart + 8 * i);
    }
  }
  const int vpart = tid & 7, vrow = tid >> 3;
  bf16x8 vv[VDP][VCH];
#pragma unroll
  for (int dp = 0; dp < VDP; ++dp)
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int k0 = kbeg + 64 * c + 8 * vpart;
      if (k0 < kend) vv[dp][c] = load_bf16x8(V1 + (long)(k0 >> 5) * (32 * HD) + (64 * dp + vrow) * 32 + (k0 & 31));
    }
  // query rows q = r GQ + j (head g GQ + j, row r) into LDS
  for (int i = tid; i < NQ * (HD / 8); i += kDecThreads) {
    const int q = i / (HD / 8), c = i % (HD / 8);
    bf16x8 v;
    if (q < nq) {
      const int h = g * GQ + q % GQ, r = q / GQ;
      v = load_bf16x8(a.q + ((long)(b * R + r) * a.H + h) * HD + 8 * c);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.f;
    }
    *reinterpret_cast<bf16x8*>(&Qs[q * HD + 8 * c]) = v;
  }
  __syncthreads();

  // scores (raw dot products; -inf where a row may not see the key)
#pragma unroll
  for (int ps = 0; ps < 4; ++ps) {
    const int kl = ps * KPP + kslot, key = kbeg + kl;
    float sc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float acc = 0.f;
      if (key < kend) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 qv = *reinterpret_cast<const bf16x8*>(&Qs[q * HD + 32 * kpart + 8 * i]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 x = {kv[ps][i][2 * e], kv[ps][i][2 * e + 1]};
            const bf16x2 y = {qv[2 * e], qv[2 * e + 1]};
            acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
          }
        }
      }
      sc[q] = acc;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1) sc[q] += __shfl_xor(sc[q], o, 64);
    if (kpart == 0) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const bool vis = key < kend && q < nq && key <= qpos0 + q / GQ;
        Ps[q * MAXK + kl] = vis ? sc[q] : -INFINITY;
      }
    }
  }
  __syncthreads();

  // softmax of row q = wave over the split (log2 units, as the MFMA kernel)
  const float sl2 = a.scale * 1.4426950408889634f;
  __shared__ float mls[NQ][2];
  const int nk = max(kend - kbeg, 0);
  if (wave < NQ) {
    const int q = wave;
    float mx = -INFINITY;
    for (int k = lane; k < nk; k += 64) mx = fmaxf(mx, Ps[q * MAXK + k]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float m2 = mx * sl2;
    float l = 0.f;
    for (int k = lane; k < MAXK; k += 64) {
      const float sv = Ps[q * MAXK + k];
      const float pv = (k < nk && mx != -INFINITY) ? __builtin_amdgcn_exp2f(fmaf(sv, sl2, -m2)) : 0.f;
      Ps[q * MAXK + k] = pv;
      l += pv;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
    if (lane == 0) {
      mls[q][0] = m2;
      mls[q][1] = l;
    }
  }
  __syncthreads();

  // O = P V over the split, normalised by the split's sum
  float o[VDP][NQ];
#pragma unroll
  for (int dp = 0; dp < VDP; ++dp)
#pragma unroll
    for (int q = 0; q < NQ; ++q) o[dp][q] = 0.f;
#pragma unroll
  for (int c = 0; c < VCH; ++c) {
    if (kbeg + 64 * c + 8 * vpart < kend) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float4 p0 = *reinterpret_cast<const float4*>(&Ps[q * MAXK + 64 * c + 8 * vpart]);
        const float4 p1 = *reinterpret_cast<const float4*>(&Ps[q * MAXK + 64 * c + 8 * vpart + 4]);
        const float pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int dp = 0; dp < VDP; ++dp) {
          float acc = o[dp][q];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf(pw[e], (float)vv[dp][c][e], acc);
          o[dp][q] = acc;
        }
      }
    }
  }
  const long BR = (long)a.B * R;
#pragma unroll
  for (int dp = 0; dp < VDP; ++dp)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float v = o[dp][q];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      if (vpart == 0 && q < nq) {
        const int h = g * GQ + q % GQ, r = q / GQ, d = 64 * dp + vrow;
        const float l = mls[q][1];
        const float y = l > 0.f ? v / l : 0.f;
        bf16_t* op = a.splits == 1 ? a.out + ((long)(b * R + r) * a.H + h) * HD
                                   : a.opart + (((long)split * BR + (long)b * R + r) * a.H + h) * HD;
        op[d] = f2bf(y);
      }
    }
  if (a.splits > 1 && tid < nq) {
    const int q = tid, h = g * GQ + q % GQ, r = q / GQ;
    float* mp = a.mlpart + (((long)split * BR + (long)b * R + r) * a.H + h) * 2;
    mp[0] = mls[q][0];
    mp[1] = mls[q][1];
  }
}

template <int HD>
static bool attn_decode(const AttnArgs& a, hipStream_t s) {
  const int nq = a.rows_per_batch * (a.H / a.Hkv);
  if (!a.causal || a.n2 != 0 || nq > 8 || a.split_len > dec_max_keys(HD)) return false;
  const dim3 grid(a.B * a.Hkv * a.splits), block(kDecThreads);
  if (nq <= 1) hipLaunchKernelGGL((attn_decode_kernel<HD, 1>), grid, block, 0, s, a);
  else if (nq <= 2) hipLaunchKernelGGL((attn_decode_kernel<HD, 2>), grid, block, 0, s, a);
  else if (nq <= 4) hipLaunchKernelGGL((attn_decode_kernel<HD, 4>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((attn_decode_kernel<HD, 8>), grid, block, 0, s, a);
  return true;
}

hipError_t attention(const AttnArgs& a, hipStream_t s) {
  const int GQ = a.H / a.Hkv;
  if (a.H % a.Hkv != 0 || (GQ != 1 && GQ != 2 && GQ != 4)) return hipErrorInvalidValue;
  if (a.split_len % 32 != 0 || a.rows_per_batch <= 0 || a.n1 % 32 != 0 || a.n2 % 32 != 0) return hipErrorInvalidValue;
  if (a.pos_dev && (!a.causal || a.n2 != 0)) return hipErrorInvalidValue;
  if (a.splits < 1 || (a.splits == 1 && !a.out) || (a.splits > 1 && (!a.opart || !a.mlpart)))
    return hipErrorInvalidValue;
  // decoding passes (a few rows per sequence, causal prefix only)
  if (a.hd == 64 ? attn_decode<64>(a, s) : a.hd == 128 ? attn_decode<128>(a, s) : a.hd == 256 && attn_decode<256>(a, s))
    return hipGetLastError();
  switch (a.hd * 10 + GQ) {
    case 641: attn_shape<64, 1>(a, s); break;
    case 642: attn_shape<64, 2>(a, s); break;
    case 644: attn_shape<64, 4>(a, s); break;
    case 1281: attn_shape<128, 1>(a, s); break;
    case 1282: attn_shape<128, 2>(a, s); break;
    case 1284: attn_shape<128, 4>(a, s); break;
    case 2561: attn_shape<256, 1>(a, s); break;
    case 2562: attn_shape<256, 2>(a, s); break;
    case 2564: attn_shape<256, 4>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dg
