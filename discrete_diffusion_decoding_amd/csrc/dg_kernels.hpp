// Launch interface of libdg's HIP kernels (host side).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_common.hpp"

namespace dg {

enum Epi { EPI_STORE_BF16 = 0, EPI_STORE_F32 = 1, EPI_GEGLU_BF16 = 4 };

// C[r, n] (op)= sum_k A[row(r), k] * W_g[n, k] over row chunks ("items").
// A: bf16 rows of pitch lda; row(r) = a_rows ? a_rows[r] : r.
// W: bf16 [N, ldw] per group, groups w_gstride elements apart (W2 likewise for GEGLU).
// Items: with `items` (device int4 {group, first row, row count, 0}, count in
// *n_items), each item is one chunk of <= 64 rows of one group; without, the
// rows [0, M) of group 0 are cut into chunks of 64.  items_max bounds the item
// count (the grid is items_max x column tiles x k_split; spare workgroups exit).
// Split-K: `k_split` ranges of `k_chunk`, partial outputs c_kstride apart.
struct GemmArgs {
  const bf16_t* A;
  long lda;
  const int32_t* a_rows;
  const bf16_t* W;
  const bf16_t* W2;
  long ldw;
  long w_gstride;
  int K, N;
  int k_chunk;
  const int4* items;
  const int32_t* n_items;
  int items_max;
  int M;
  int k_split;
  int tile_rows;   // 64-row kernel: activation rows per tile (64, the work-list chunk size; dense rows also 128),
  int tile_cols;   // weight rows per tile (64 | 128)
  int ring;        // and its LDS ring depth (64 wide: 4 | 5; 128 wide: 2 | 3)
  int few_rows;    // work-list products: a bound (1..kGemvRows) on the rows of every item, when one is
                   // known (decoding); 0 otherwise.  Dense products use M.
  int waves8;      // dense store products: the 8-wave tile kernel (two waves per SIMD)
  // GEMV work lists only: items of group >= grp_x read Wx (GEGLU up: Wx2) +
  // (group - grp_x) * wx_gstride, rows ldwx apart (the shared FFN's blocks as
  // extra experts); Wx == nullptr: none
  const bf16_t* Wx;
  const bf16_t* Wx2;
  long ldwx, wx_gstride;
  int grp_x;
  void* C;
  long ldc;
  long c_kstride;
  const int32_t* flag;
};

hipError_t gemm(int epi, const GemmArgs& a, hipStream_t s);
// 256 activation rows x 128 weight rows per workgroup; dense rows only (items_max =
// ceil(M / 256)); epilogues EPI_STORE_F32 (split-K partials) and EPI_STORE_BF16
hipError_t gemm_fat(int epi, const GemmArgs& a, hipStream_t s);
hipError_t gemm_fat2(int epi, const GemmArgs& a, hipStream_t s);
// C [M][N] fp32 split-K partials = A [M][K] W [K][N] (W K-major), 256 x 256 tiles
hipError_t gemm_kn(const GemmArgs& a, hipStream_t s);
constexpr int kFatRowChunk = 256;
// the 256-row kernel addresses a tile with 32-bit byte offsets from its first row
inline bool gemm_fat_pitch_ok(long lda, long ldw) {
  return (long)kFatRowChunk * lda * 2 < 0x7FFFFFFFL && 128L * ldw * 2 < 0x7FFFFFFFL;
}
inline bool gemm_fat2_pitch_ok(long lda, long ldw) {
  return (long)kFatRowChunk * lda * 2 < 0x7FFFFFFFL && 256L * ldw * 2 < 0x7FFFFFFFL;
}
constexpr int kGemmRowChunk = 64;
// products whose items hold at most kGemvRows rows (and k chunks of at most
// kGemvK columns) run on the weight-streaming GEMV kernel instead
constexpr int kGemvRows = 4;
constexpr int kGemvK = 4096;

// ---- elementwise / reduction kernels (k_elem.hip) ----

hipError_t embed_rows(const int32_t* tokens, const bf16_t* E, int rows, int d, float* h,
                      const int32_t* flag, hipStream_t s);
// Split-K partial sums: nsplit slices `stride` floats apart, each [rows][d] (or [rows][E]).
struct Partials {
  const float* p;
  int n;
  long stride;
};

// h += (gate ? sigmoid(gate) : 1) * sum_s part_s (optional); out = bf16(rms(h) * w);
// optional hi/lo split rows for the router, optional dump of h
hipError_t rmsnorm_rows(float* h, const bf16_t* w, int rows, int d, float eps, bf16_t* out, bf16_t* split_hi_lo,
                        float* dump, Partials part, const bf16_t* part_gate, const int32_t* flag, hipStream_t s);
// per-head RMSNorm + RoPE of q and k, scatter of k / v into the attention caches
struct QkRopeArgs {
  const bf16_t* qkv; int rows; int H, Hkv, hd; float eps; float theta;
  const float2* rope;               // [per_batch][hd/2] (cos, sin) from rope_table
  const bf16_t* qnorm; const bf16_t* knorm;
  bf16_t* q;                        // [rows][H][hd]
  int per_batch, pos0;              // position of row r = pos0 + (r % per_batch)
  bf16_t* kdst; long k_bstride, k_hstride;            // K rows [.][Hkv][pitch][hd]
  bf16_t* vtdst; long v_bstride, v_hstride;  // V^T [.][Hkv][positions / 32][hd][32] (tile-major)
  int t_offset;                     // index of row 0 within the destination sequence
  const int32_t* pos_dev;           // if set: t_offset read from the device
  const int32_t* flag;
};
hipError_t qk_norm_rope(const QkRopeArgs& a, hipStream_t s);
// pos_dev (may be null): pos0 read from the device instead
hipError_t rope_table(float2* tab, int per_batch, int pos0, int hd, float theta, const int32_t* pos_dev,
                      hipStream_t s);

struct AttnArgs {
  const bf16_t* q; int H, Hkv, hd; float scale;
  int rows_per_batch; int B;
  // key source 1 (cache) and 2 (canvas); batch b reads source-1 element b1 = (nb1 == 1 ? 0 : b)
  // (V^T tile-major: [keys / 32][hd][32] from each head's base)
  const bf16_t* k1; const bf16_t* vt1; long k1_bstride, k1_hstride, v1_bstride, v1_hstride; int n1; int nb1;
  const bf16_t* k2; const bf16_t* vt2; long k2_bstride, k2_hstride, v2_bstride, v2_hstride; int n2;
  int causal; int qpos0;            // causal: query row r (within batch) sits at qpos0 + r
  int splits; int split_len;        // key splits (split_len multiple of 32)
  const int32_t* pos_dev;           // causal pass (n2 = 0) whose first query position is read from the
                                    // device: qpos0 = *pos_dev, n1 = that + rows rounded up to 32 keys
  bf16_t* out;                      // one split: O [B*rows][H][hd] (bf16, normalised)
  bf16_t* opart; float* mlpart;     // more: per split normalised O [splits][B*rows][H][hd] (bf16)
                                    // and (running max in log2 units, sum) [splits][B*rows][H][2]
  const int32_t* flag;
};
hipError_t attention(const AttnArgs& a, hipStream_t s);
// attention workgroup shape: attn_waves(hd) waves of attn_frags(hd) row
// fragments (16 rows) each, i.e. 16 * waves * frags (query, head) rows
constexpr int attn_waves(int hd) { return hd >= 256 ? 8 : 4; }
constexpr int attn_frags(int hd) { return hd >= 256 ? 1 : hd >= 128 ? 2 : 4; }
constexpr int attn_rows_per_wg(int hd) { return 16 * attn_waves(hd) * attn_frags(hd); }
hipError_t attention_merge(const bf16_t* opart, const float* mlpart, int splits, int rows, int H, int hd,
                           bf16_t* out, const int32_t* flag, hipStream_t s);

// router logits = sum over split-K partials of the hi rows [0, rows) and lo rows [rows, 2 rows)
// idx / gate [rows][k + ns]: the top-k, then experts E .. E + ns - 1 with gate 1;
// logit_dump (optional) [rows][E]: the summed logits
hipError_t router_topk(Partials rlog, int rows, int E, int k, int ns, int32_t* idx, float* gate, int32_t* idx_dump,
                       float* gate_dump, float* logit_dump, const int32_t* flag, hipStream_t s);
// at most 4 rows: router_topk then moe_permute (chunk >= rows) in one launch
hipError_t router_topk_permute(Partials rlog, int rows, int E, int k, int ns, int32_t* idx, float* gate,
                               int32_t* idx_dump, float* gate_dump, float* logit_dump, int32_t* counts, int32_t* offsets,
                               int32_t* slot_of, int32_t* slot_row, int4* items, int32_t* n_items, int chunk,
                               const int32_t* flag, hipStream_t s);
// k values moe_combine takes
inline bool combine_k_ok(int k) { return k == 1 || k == 2 || k == 4 || k == 8 || k == 11; }
// also emits the GEMM work list: int4 {expert, first slot, rows, chunk index << 16 |
// chunks of the expert} per chunk of <= chunk rows of every touched expert, and
// its length in *n_items
hipError_t moe_permute(const int32_t* idx, int rows, int k, int E, int32_t* counts, int32_t* offsets,
                       int32_t* slot_of, int32_t* slot_row, int4* items, int32_t* n_items, int chunk,
                       const int32_t* flag, hipStream_t s);
// h[r] += sum_s ys_s[r] + sum_j gate[r,j] * Y[slot_of[r,j]]; then optional next RMSNorm -> xn, dump of h
hipError_t moe_combine(float* h, Partials ys, const bf16_t* Y, const int32_t* slot_of, const float* gate,
                       int rows, int d, int k, const bf16_t* next_w, float eps, bf16_t* xn, float* dump,
                       const int32_t* flag, hipStream_t s);

// ---- LM head / sampler (k_head.hip) ----
struct SampleArgs {
  const float* logits; int B, T, V; long ldl;
  int step_arg;                     // >= 0: this step; < 0: read steps[b]
  float tau_start, tau_end; int max_steps;
  int lock_rule; float lock_thresh; int stop_rule; float stop_thresh;
  uint64_t seeds[16];
  int vsplit;                       // vocab slices per row
  float* part;                      // [B*T][vsplit][8]
  float4* rowstat;                  // [B*T] out (optional): max, Z, entropy, argmax (int bits)
  // the softmax statistics computed by the vocabulary-tiled LM head (same
  // layout as rowstat): when set, the partial pass keeps only the Gumbel
  // maximum and the finishing pass takes entropy and argmax from here
  const float4* rowstat_in;
  int32_t* tokens; uint8_t* locked; float* entropy; int32_t* xhat; int32_t* argmax;
  int32_t* stopped; int32_t* steps; int32_t* all_stopped;
  const int32_t* flag;
};
// autoregressive next-token sample: B rows of V logits (row pitch ldl), one
// decode position; V and ldl multiples of 4
struct ArSampleArgs {
  const float* logits; int B, V; long ldl;
  float inv_tau; int pos;
  const int32_t* pos_dev;           // if set: pos read from the device
  uint64_t seeds[16];
  int vsplit;                       // vocab slices per row
  float* part;                      // [B][vsplit][8]
  int32_t* next; int32_t* argmax; float* entropy;   // [B]; argmax / entropy may be null
};
hipError_t ar_sample(const ArSampleArgs& a, hipStream_t s);
hipError_t sample_partial(const SampleArgs& a, hipStream_t s);
hipError_t sample_finish(const SampleArgs& a, hipStream_t s);
// The vocabulary in nslices slices of kchunk entries (the split of the
// soft-prediction product's contraction).  Per (row, slice): the slice's
// softmax statistics {max m_s, Z_s = sum e^(l - m_s), A_s = sum e^(l - m_s)(l - m_s),
// argmax} into sstat [rows][nslices], and (P not null) the slice-scaled
// probabilities P[r][v] = bf16(e^(l_v - m_s)).  Rows of canvases stopped on
// entry (stopped[r / T]) are skipped.
hipError_t softmax_slices(const float* logits, long ldl, int rows, int V, int kchunk, int nslices, int T,
                          const int32_t* stopped, bf16_t* P, float4* sstat, const int32_t* flag, hipStream_t s);
// Per row: the slice statistics merged (online softmax) into rowstat {max, Z,
// entropy ln Z - A / Z, argmax}; with part (the soft-prediction product's
// split-K partials [nslices][rows][d]), also out[r] = bf16(sum_s e^(m_s - M) / Z
// part[s][r]).  Rows of stopped canvases are skipped.
hipError_t softmax_finish(const float4* sstat, int nslices, int rows, int T, const int32_t* stopped,
                          const float* part, int d, bf16_t* out, float4* rowstat, const int32_t* flag, hipStream_t s);
hipError_t init_canvas(int32_t* tokens, int B, int T, int V, const uint64_t* seeds, hipStream_t s);
hipError_t fill_i32(int32_t* p, int32_t v, long n, hipStream_t s);
hipError_t fill_u16(uint16_t* p, uint16_t v, long n, hipStream_t s);
hipError_t set_step(int32_t* steps, const int32_t* stopped, int B, int step, hipStream_t s);

}  // namespace dg
