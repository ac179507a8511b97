// libdg host runtime: argument checks, workspace planning and the launch
// sequence of the denoising step (C ABI declared in include/dg.h).
//
// Step structure (DiffusionGemma, laozijiushiniubi article sections 2 and 4):
//   embed canvas tokens (+ gated self-conditioning projection of s_prev)
//   for each layer: RMSNorm -> QKV -> QK-norm + RoPE -> attention over
//     (cached prefix, bidirectional canvas) -> O projection + residual ->
//     RMSNorm -> router top-k -> expert permutation -> grouped expert FFNs
//     (+ shared FFN) -> weighted combine + residual (fused with the next norm)
//   final norm -> LM head -> entropy / Gumbel-max / lock / re-randomise / stop
//   -> soft-prediction embedding s_next = softmax(logits) E
// Nothing here allocates device memory; every buffer is carved out of the
// caller's workspace.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "dg.h"
#include "dg_kernels.hpp"
#include "dg_rng.hpp"

using namespace dg;

// Optional per-kernel-class timing with HIP events (off by default).
struct Prof {
  bool on = false;
  std::vector<hipEvent_t> pool;   // event pairs, reused across calls
  std::vector<int> cls;           // class of each recorded pair
  size_t used = 0;
};

// A captured step (one hipGraph per distinct set of step arguments).
struct GraphKey {
  int kind;  // 0: dg_denoise_step, 1: a step of dg_generate_block (stop-flag early exits), 2: dg_ar_step
  const void* kv;
  int Bp, P, P_max, B, T;
  dg_canvas c;
  float tau_start, tau_end, lock_thresh, stop_thresh;
  int max_steps, lock_rule, stop_rule;
  uint64_t seeds[16];
  void* ws;
  size_t ws_bytes;
};

struct GraphEntry {
  GraphKey key;
  hipGraphExec_t exec;
  unsigned long long last_use;
};

struct dg_model {
  dg_model_desc d;
  dg_weights w;
  std::vector<const bf16_t*> layers;
  dg_layer_layout lay;
  mutable Prof prof;
  bool use_graphs = true;
  // 64-row GEMM kernel variants: grouped expert products (tile rows, ring) and dense (ring)
  int x_rows = 64, x_cols = 64, x_ring = 5, d_ring = 4;
  // expert down projection: 128 weight rows per tile (22 tiles of d), double
  // buffered so three workgroups share a CU (its K is only 11 stages long)
  int xd_cols = 128, xd_ring = 2;
  // second stream (default priority) for the shared FFN, which runs beside the
  // routed path; created on first use, with its fork / join events
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  bool side_failed = false;
  std::vector<GraphEntry> graphs;
  unsigned long long use_clock = 0;
};

// timing scope: records an event pair around the enclosed launches when on
struct ProfScope {
  Prof& p;
  hipStream_t st;
  size_t idx;
  bool rec;
  ProfScope(const dg_model* m, int c, hipStream_t s) : p(m->prof), st(s), idx(0), rec(false) {
    if (!p.on) return;
    if (p.used * 2 + 2 > p.pool.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return;
      p.pool.push_back(a);
      p.pool.push_back(b);
      p.cls.push_back(c);
    }
    idx = p.used++;
    p.cls[idx] = c;
    rec = hipEventRecord(p.pool[2 * idx], st) == hipSuccess;
  }
  ~ProfScope() {
    if (rec) (void)hipEventRecord(p.pool[2 * idx + 1], st);
  }
};

#define DG_CK(x)                                                        \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) {                                             \
      fprintf(stderr, "libdg: %s failed: %s\n", #x, hipGetErrorString(e_)); \
      return DG_ERR_HIP;                                                \
    }                                                                   \
  } while (0)

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
static size_t al128e(size_t x) { return (x + 127) & ~(size_t)127; }
static int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

extern "C" const char* dg_status_string(dg_status s) {
  switch (s) {
    case DG_OK: return "ok";
    case DG_ERR_ARG: return "invalid argument";
    case DG_ERR_SHAPE: return "unsupported shape";
    case DG_ERR_WORKSPACE: return "workspace too small";
    case DG_ERR_HIP: return "HIP error";
    case DG_ERR_UNSUPPORTED: return "unsupported request";
  }
  return "unknown status";
}

static dg_status check_desc(const dg_model_desc* d) {
  if (!d) return DG_ERR_ARG;
  if (d->n_layers < 1 || d->d_model < 64 || d->n_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
      d->n_experts < 1 || d->top_k < 1 || d->d_expert < 1 || d->d_shared < 0 || d->vocab < 0 ||
      (d->self_cond != 0 && d->self_cond != 1) || !(d->rms_eps >= 0.f) || !(d->rope_theta > 0.f))
    return DG_ERR_ARG;
  const int gq = d->n_heads % d->n_kv_heads == 0 ? d->n_heads / d->n_kv_heads : 0;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return DG_ERR_SHAPE;
  if (gq != 1 && gq != 2 && gq != 4) return DG_ERR_SHAPE;
  if (d->d_model % 64 || d->d_model > 4096 || d->d_expert % 64 || d->d_shared % 64 ||
      (d->n_heads * d->head_dim) % 64)
    return DG_ERR_SHAPE;
  if (d->n_experts > 255 || d->top_k > d->n_experts) return DG_ERR_SHAPE;
  if (d->top_k != 1 && d->top_k != 2 && d->top_k != 4 && d->top_k != 8) return DG_ERR_SHAPE;
  if (d->vocab % 128) return DG_ERR_SHAPE;
  if (d->self_cond && d->vocab == 0) return DG_ERR_SHAPE;
  return DG_OK;
}

extern "C" dg_status dg_layer_layout_get(const dg_model_desc* d, dg_layer_layout* o) {
  dg_status st = check_desc(d);
  if (st != DG_OK) return st;
  if (!o) return DG_ERR_ARG;
  const size_t D = d->d_model, hd = d->head_dim, E = d->n_experts, fe = d->d_expert, fs = d->d_shared;
  const size_t qkv = (size_t)(d->n_heads + 2 * d->n_kv_heads) * hd;
  size_t p = 0;
  auto take = [&](size_t n) { size_t r = p; p = al128e(p + n); return r; };
  o->attn_norm = take(D);
  o->w_qkv = take(qkv * D);
  o->q_norm = take(hd);
  o->k_norm = take(hd);
  o->w_o = take(D * d->n_heads * hd);
  o->ffn_norm = take(D);
  o->w_router = take(E * D);
  o->w_gate = take(E * fe * D);
  o->w_up = take(E * fe * D);
  o->w_down = take(E * D * fe);
  o->w_gate_sh = take(fs * D);
  o->w_up_sh = take(fs * D);
  o->w_down_sh = take(D * fs);
  o->total = p;
  return DG_OK;
}

extern "C" dg_status dg_model_create(const dg_model_desc* d, const dg_weights* w, dg_model** out) {
  dg_status st = check_desc(d);
  if (st != DG_OK) return st;
  if (!w || !out || !w->layers) return DG_ERR_ARG;
  if (d->vocab && (!w->embed || !w->final_norm)) return DG_ERR_ARG;
  if (d->self_cond && (!w->self_cond_w || !w->self_cond_gate)) return DG_ERR_ARG;
  for (int l = 0; l < d->n_layers; ++l)
    if (!w->layers[l]) return DG_ERR_ARG;
  dg_model* m = new dg_model();
  m->d = *d;
  m->w = *w;
  m->layers.resize(d->n_layers);
  for (int l = 0; l < d->n_layers; ++l) m->layers[l] = (const bf16_t*)w->layers[l];
  m->w.layers = nullptr;
  dg_layer_layout_get(d, &m->lay);
  *out = m;
  return DG_OK;
}

extern "C" void dg_model_destroy(dg_model* m) {
  if (!m) return;
  if (m->side) (void)hipStreamDestroy(m->side);
  if (m->ev_fork) (void)hipEventDestroy(m->ev_fork);
  if (m->ev_join) (void)hipEventDestroy(m->ev_join);
  for (hipEvent_t e : m->prof.pool) (void)hipEventDestroy(e);
  for (GraphEntry& g : m->graphs) (void)hipGraphExecDestroy(g.exec);
  delete m;
}

extern "C" dg_status dg_set_graphs(dg_model* m, int32_t enable) {
  if (!m) return DG_ERR_ARG;
  m->use_graphs = enable != 0;
  return DG_OK;
}

extern "C" size_t dg_kv_bytes(const dg_model* m, int32_t Bp, int32_t P_max) {
  if (!m || Bp < 1 || P_max < 0) return 0;
  const dg_model_desc& d = m->d;
  return (size_t)d.n_layers * 2 * Bp * d.n_kv_heads * (size_t)P_max * d.head_dim * sizeof(bf16_t);
}

// ---------------------------------------------------------------------------
// workspace plan
struct Plan {
  size_t h, xn, qkv, q, kc, vc, rope, opart, ml, o, dpart, xn2, xr, rlog, eidx, egate, cnt, off, slot_of, slot_row, items,
      nitems, hbuf, ybuf, hs, ys, logits, spart, sstat, rowstat, P, separt, flag, pos, total;
  int splits_max, vsplit, ksplit, kchunk;
};

static const int kMaxSplits = 16;
static const int kMaxDenseSplit = 8;    // split-K slices of a dense projection
static const int kMaxRouterSplit = 8;   // split-K slices of the router logits

// Split-K slices for the 64-row kernel (two workgroups per CU); returns the
// slice count and sets the 64-aligned slice length: the count that minimises the modelled time, workgroup length (its 64-column stages plus
// a fixed cost of 4 for fill and epilogue) times the rounds the grid needs on
// 256 CUs (a full round of 512 takes two lengths; a remainder of up to 256
// takes one); ties go to fewer slices (fewer partial sums).
static int choose_ksplit(long tiles_times_items, int K, int max_split, int* k_chunk) {
  const long t = std::max(1L, tiles_times_items);
  int best_ks = 1, best_kc = cdiv(K, 64) * 64;
  long best_time = -1;
  const int top = std::max(1, std::min(max_split, K / 128));
  for (int want = 1; want <= top; ++want) {
    const int kc = cdiv(cdiv(K, want), 64) * 64;
    const int ks = cdiv(K, kc);
    const long n = t * ks, w = kc / 64 + 4;
    const long full = n / 512, rem = n % 512;
    const long time = w * (2 * full + (rem + 255) / 256);
    if (best_time < 0 || time < best_time) {
      best_time = time;
      best_ks = ks;
      best_kc = kc;
    }
  }
  *k_chunk = best_kc;
  return best_ks;
}

// Products with at least this many rows run on the 256 x 256 tile kernel:
// every weight byte then enters one workgroup only (the 64-row kernel fetches
// it once per 64-row chunk), and every activation byte fetched feeds 256
// weight rows.
static const int kFatMinRows = 192;
static bool fat_rows(int rows) { return rows >= kFatMinRows; }

// dense store products of at least this many rows take the 8-wave tile kernel
// (measured at 256 rows: 9.37 -> 9.28 ms per full step)
static const int kWaves8MinRows = 128;

// Soft-embedding product (K = vocab, 256 x 256 tiles of the K-major kernel):
// split so that ~256 workgroups (one per CU, at most one round) share the
// contraction.
static void soft_split(const dg_model_desc& d, int rows, int* ksplit, int* kchunk) {
  const int items = cdiv(d.d_model, 256) * cdiv(rows, 256);
  int ks = std::max(1, std::min(32, 256 / items));
  int kc = cdiv(cdiv(d.vocab, ks), 64) * 64;
  *kchunk = kc;
  *ksplit = cdiv(d.vocab, kc);
}

// Dense product C = A W^T over rows [0, M) on the kernel suited to M.
static hipError_t dense_gemm(int epi, GemmArgs g, int M, hipStream_t st) {
  g.M = M;
  g.items = nullptr;
  g.n_items = nullptr;
  if (fat_rows(M) && (epi == EPI_STORE_F32 || epi == EPI_STORE_BF16) && !g.a_rows &&
      gemm_fat_pitch_ok(g.lda, g.ldw)) {
    g.items_max = cdiv(M, kFatRowChunk);
    if (gemm_fat2_pitch_ok(g.lda, g.ldw)) return gemm_fat2(epi, g, st);
    return gemm_fat(epi, g, st);
  }
  g.items_max = cdiv(M, kGemmRowChunk);
  g.waves8 = M >= kWaves8MinRows && g.tile_rows == 64 && g.tile_cols == 64 && g.ring == 4;
  return gemm(epi, g, st);
}

static int vsplit_of(int rows, int V) {
  const int groups = std::max(1, rows / 4);
  int vs = std::max(1, std::min(64, cdiv(2048, groups)));
  while (vs > 1 && V / vs < 1024) vs >>= 1;
  return vs;
}

// Decoding (at most kGemvRows rows): the shared FFN runs as d_shared / d_expert
// extra experts E .. E + ns - 1 that every row takes with gate 1, inside the
// grouped GEMV products (no second stream, no fork / join).  Returns ns, or 0
// when the shared FFN runs as its own dense products.
static int shared_as_experts(const dg_model_desc& d, int rows) {
  if (d.d_shared == 0 || rows > kGemvRows || d.d_shared % d.d_expert) return 0;
  const int ns = d.d_shared / d.d_expert;
  if (d.n_experts + ns > 255 || !combine_k_ok(d.top_k + ns)) return 0;
  return ns;
}

static Plan make_plan(const dg_model_desc& d, int rows, int keys) {
  Plan p{};
  const size_t R = rows, D = d.d_model, hd = d.head_dim, H = d.n_heads, Hkv = d.n_kv_heads, E = d.n_experts,
               k = d.top_k, V = d.vocab;
  const size_t qkvd = (H + 2 * Hkv) * hd;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = al256(o + bytes); return r; };
  (void)keys;
  p.splits_max = kMaxSplits;
  p.h = take(R * D * 4);
  p.xn = take(R * D * 2);
  p.qkv = take(R * qkvd * 2);
  p.q = take(R * H * hd * 2);
  p.kc = take(R * Hkv * hd * 2);
  p.vc = take(R * Hkv * hd * 2);
  p.rope = take(R * (hd / 2) * 8);
  p.opart = take((size_t)kMaxSplits * R * H * hd * 2);
  p.ml = take((size_t)kMaxSplits * R * H * 2 * 4);
  p.o = take(R * H * hd * 2);
  p.dpart = take((size_t)kMaxDenseSplit * R * D * 4);
  p.xn2 = take(R * D * 2);
  p.xr = take(2 * R * D * 2);
  p.rlog = take((size_t)kMaxRouterSplit * 2 * R * E * 4);
  // expert slots: top-k per row, plus the shared FFN's blocks in passes of at
  // most kGemvRows rows (any pass this workspace serves may be one)
  const size_t ns = shared_as_experts(d, 1), Ex = E + ns;
  const size_t slots = std::max(R * k, std::min(R, (size_t)kGemvRows) * (k + ns));
  p.eidx = take(slots * 4);
  p.egate = take(slots * 4);
  p.cnt = take((Ex + 1) * 4);
  p.off = take((Ex + 1) * 4);
  p.slot_of = take(slots * 4);
  p.slot_row = take(slots * 4);
  p.items = take((Ex + (slots + 31) / 32) * 16);   // work list for chunks of >= 32 rows
  p.nitems = take(16);
  p.hbuf = take(slots * d.d_expert * 2);
  p.ybuf = take(slots * D * 2);
  p.hs = take(R * std::max(d.d_shared, 1) * 2);
  p.ys = take(d.d_shared ? (size_t)kMaxDenseSplit * R * D * 4 : 0);
  if (V) {
    p.vsplit = vsplit_of(rows, (int)V);
    p.logits = take(R * V * 4);
    p.spart = take(R * p.vsplit * 8 * 4);
    // vocabulary slices: the split of the soft-prediction product's contraction
    soft_split(d, rows, &p.ksplit, &p.kchunk);
    p.sstat = take(R * p.ksplit * 16);
    p.rowstat = take(R * 16);
    if (d.self_cond) {
      p.P = take(R * V * 2);
      p.separt = take((size_t)p.ksplit * R * D * 4);
    }
  }
  p.flag = take(64);
  p.pos = take(64);
  p.total = o;
  return p;
}

extern "C" size_t dg_workspace_bytes(const dg_model* m, int32_t rows, int32_t keys) {
  if (!m || rows < 1 || keys < 0) return 0;
  return make_plan(m->d, rows, keys).total;
}

template <class T>
static T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

// ---------------------------------------------------------------------------
struct Pass {
  int rows, B, per_batch, pos0;
  bool prefill;
  int bp, q0;                 // prefill: prefix index, first position of the chunk
  const bf16_t* kv;           // cache base
  int kv_Bp;                  // prefixes held by the cache (layer stride)
  int Bp, P, P_max;           // step: prefix batch, prefix length, capacity
  float* hidden_dump;
  int32_t* expert_dump;
  float* gate_dump;
  float* router_dump;
  bool final_norm;            // last combine writes the final-normed hidden into xn
  const int32_t* flag;
  const int32_t* pos_dev;     // prefill of one position read from the device (q0, pos0 unused)
};

static const bf16_t* lw(const dg_model* m, int l, size_t off) { return m->layers[l] + off; }


static GemmArgs gargs() {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.k_split = 1;
  g.tile_rows = 64;
  g.tile_cols = 64;
  g.ring = 4;
  return g;
}

// dense rows [0, M) in chunks of kGemmRowChunk
static void dense_rows(GemmArgs& g, int M) {
  g.M = M;
  g.items = nullptr;
  g.n_items = nullptr;
  g.items_max = cdiv(M, kGemmRowChunk);
}

// the side stream, created on first use; false (run serially) if it cannot be made
static bool side_stream(const dg_model* mc) {
  dg_model* m = const_cast<dg_model*>(mc);
  if (m->side) return true;
  if (m->side_failed) return false;
  if (hipStreamCreateWithFlags(&m->side, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&m->ev_fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&m->ev_join, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    m->side_failed = true;
    if (m->side) (void)hipStreamDestroy(m->side);
    m->side = nullptr;
    return false;
  }
  return true;
}

static dg_status run_layers(const dg_model* m, const Plan& p, void* ws, const Pass& ps, hipStream_t st) {
  const dg_model_desc& d = m->d;
  const int R = ps.rows, D = d.d_model, H = d.n_heads, Hkv = d.n_kv_heads, hd = d.head_dim, E = d.n_experts,
            k = d.top_k, fe = d.d_expert, fs = d.d_shared;
  const int qkvd = (H + 2 * Hkv) * hd;
  // cache of one layer: K [kv_Bp][Hkv][P_max][hd], then V^T [kv_Bp][Hkv][P_max / 32][hd][32]
  const size_t kv_one = (size_t)Hkv * ps.P_max * hd;  // elements of one prefix, K or V
  const size_t layer_kv = (size_t)2 * ps.kv_Bp * kv_one;
  float* h = at<float>(ws, p.h);
  bf16_t* xn = at<bf16_t>(ws, p.xn);
  bf16_t* qkv = at<bf16_t>(ws, p.qkv);
  bf16_t* q = at<bf16_t>(ws, p.q);
  bf16_t* o = at<bf16_t>(ws, p.o);
  bf16_t* xn2 = at<bf16_t>(ws, p.xn2);
  bf16_t* xr = at<bf16_t>(ws, p.xr);
  float* rlog = at<float>(ws, p.rlog);
  int32_t* eidx = at<int32_t>(ws, p.eidx);
  float* egate = at<float>(ws, p.egate);
  int32_t* cnt = at<int32_t>(ws, p.cnt);
  int32_t* off = at<int32_t>(ws, p.off);
  int32_t* slot_of = at<int32_t>(ws, p.slot_of);
  int32_t* slot_row = at<int32_t>(ws, p.slot_row);
  int4* items = at<int4>(ws, p.items);
  int32_t* nitems = at<int32_t>(ws, p.nitems);
  // shared FFN blocks as experts E .. Ex - 1 (decoding), in slots k .. kx - 1 of every row
  const int ns = shared_as_experts(d, R), Ex = E + ns, kx = k + ns;
  // every item holds at least one of the R kx slots
  const int items_max = (int)std::min<long>(Ex + cdiv((long)R * kx, m->x_rows), (long)R * kx);
  bf16_t* hbuf = at<bf16_t>(ws, p.hbuf);
  bf16_t* ybuf = at<bf16_t>(ws, p.ybuf);
  bf16_t* hs = at<bf16_t>(ws, p.hs);
  float* ys = fs ? at<float>(ws, p.ys) : nullptr;

  // attention split choice: about one workgroup per CU
  const int GQ = H / Hkv;
  // (a position read on the device: the split plan covers the whole capacity,
  // and splits past the last key exit at once)
  const int nkeys = ps.prefill ? (ps.pos_dev ? ps.P_max : ps.q0 + R) : ps.P + ps.per_batch;
  const int base_wg = cdiv(ps.per_batch, attn_rows_per_wg(hd) / GQ) * Hkv * ps.B;   // per key split
  int splits = std::max(1, std::min(p.splits_max, cdiv(256, base_wg)));
  const int split_len = cdiv(cdiv(nkeys, splits), 32) * 32;
  splits = cdiv(nkeys, split_len);

  {
    ProfScope ps_(m, DG_PROF_OTHER, st);
    DG_CK(rope_table(at<float2>(ws, p.rope), ps.per_batch, ps.pos0, hd, d.rope_theta, ps.pos_dev, st));
  }
  for (int l = 0; l < d.n_layers; ++l) {
    const bf16_t* kvl = ps.kv ? ps.kv + (size_t)l * layer_kv : nullptr;
    const size_t bpo = ps.prefill ? (size_t)ps.bp * kv_one : 0;   // prefill: this prefix only
    const bf16_t* Kc = kvl ? kvl + bpo : nullptr;
    const bf16_t* Vc = kvl ? kvl + (size_t)ps.kv_Bp * kv_one + bpo : nullptr;
    // QKV
    {
      GemmArgs g = gargs();
      g.ring = m->d_ring;
      g.A = xn; g.lda = D; g.W = lw(m, l, m->lay.w_qkv); g.ldw = D; g.K = D; g.N = qkvd; g.k_chunk = D;
      dense_rows(g, R); g.C = qkv; g.ldc = qkvd; g.flag = ps.flag;
      // 128-wide weight tiles: without a k split there are enough of them at
      // 128+ rows, and each activation byte fetched then feeds twice the weight
      // rows; fewer rows (decoding) keep 64-wide tiles, twice as many workgroups
      if (R >= 128) { g.tile_cols = 128; g.ring = 3; }
      g.waves8 = R >= kWaves8MinRows;
      ProfScope ps_(m, DG_PROF_DENSE, st);
      DG_CK(gemm(EPI_STORE_BF16, g, st));
    }
    // QK norm + RoPE; K / V^T scatter
    {
      QkRopeArgs a;
      memset(&a, 0, sizeof(a));
      a.qkv = qkv; a.rows = R; a.H = H; a.Hkv = Hkv; a.hd = hd; a.eps = d.rms_eps; a.theta = d.rope_theta;
      a.qnorm = lw(m, l, m->lay.q_norm); a.knorm = lw(m, l, m->lay.k_norm); a.q = q;
      a.per_batch = ps.per_batch; a.pos0 = ps.pos0; a.flag = ps.flag; a.rope = at<float2>(ws, p.rope);
      if (ps.prefill) {
        a.kdst = const_cast<bf16_t*>(Kc); a.k_bstride = 0; a.k_hstride = (long)ps.P_max * hd;
        a.vtdst = const_cast<bf16_t*>(Vc); a.v_bstride = 0; a.v_hstride = (long)hd * ps.P_max;
        a.t_offset = ps.q0; a.pos_dev = ps.pos_dev;
      } else {
        const int T = ps.per_batch;
        a.kdst = at<bf16_t>(ws, p.kc); a.k_bstride = (long)Hkv * T * hd; a.k_hstride = (long)T * hd;
        a.vtdst = at<bf16_t>(ws, p.vc); a.v_bstride = (long)Hkv * hd * T; a.v_hstride = (long)hd * T;
        a.t_offset = 0;
      }
      ProfScope ps_(m, DG_PROF_OTHER, st);
      DG_CK(qk_norm_rope(a, st));
    }
    // attention
    {
      AttnArgs a;
      memset(&a, 0, sizeof(a));
      a.q = q; a.H = H; a.Hkv = Hkv; a.hd = hd; a.scale = 1.0f / sqrtf((float)hd);
      a.rows_per_batch = ps.per_batch; a.B = ps.B;
      a.splits = splits; a.split_len = split_len;
      a.out = o; a.opart = at<bf16_t>(ws, p.opart); a.mlpart = at<float>(ws, p.ml); a.flag = ps.flag;
      if (ps.prefill) {
        a.k1 = Kc; a.vt1 = Vc; a.k1_bstride = 0; a.k1_hstride = (long)ps.P_max * hd;
        // keys up to the last row's position, in whole 32-key tiles: the causal
        // mask hides the tail, so a pass may start and end anywhere
        a.v1_bstride = 0; a.v1_hstride = (long)hd * ps.P_max;
        a.n1 = cdiv(ps.q0 + R, 32) * 32; a.nb1 = 1;
        a.n2 = 0; a.causal = 1; a.qpos0 = ps.q0; a.pos_dev = ps.pos_dev;
      } else {
        const int T = ps.per_batch;
        if (ps.P > 0) {
          a.k1 = Kc; a.vt1 = Vc; a.k1_bstride = (long)Hkv * ps.P_max * hd; a.k1_hstride = (long)ps.P_max * hd;
          a.v1_bstride = (long)Hkv * hd * ps.P_max; a.v1_hstride = (long)hd * ps.P_max;
        } else {
          a.k1 = at<bf16_t>(ws, p.kc); a.vt1 = at<bf16_t>(ws, p.vc);
        }
        a.n1 = ps.P; a.nb1 = ps.Bp;
        a.k2 = at<bf16_t>(ws, p.kc); a.vt2 = at<bf16_t>(ws, p.vc);
        a.k2_bstride = (long)Hkv * T * hd; a.k2_hstride = (long)T * hd;
        a.v2_bstride = (long)Hkv * hd * T; a.v2_hstride = (long)hd * T; a.n2 = T;
        a.causal = 0; a.qpos0 = ps.P;
      }
      ProfScope ps_(m, DG_PROF_ATTN, st);
      DG_CK(attention(a, st));
      if (splits > 1)
        DG_CK(attention_merge(at<bf16_t>(ws, p.opart), at<float>(ws, p.ml), splits, R, H, hd, o, ps.flag, st));
    }
    // O projection: split-K partials, summed into the residual by the next norm
    Partials opp{at<float>(ws, p.dpart), 1, (long)R * D};
    {
      GemmArgs g = gargs();
      g.ring = m->d_ring;
      g.A = o; g.lda = H * hd; g.W = lw(m, l, m->lay.w_o); g.ldw = H * hd; g.K = H * hd; g.N = D;
      dense_rows(g, R);
      // 128-row activation tiles: each weight tile is streamed by half as many
      // workgroups (measured: 1 us less per layer at 256 rows than 64-row tiles)
      g.tile_rows = 128; g.ring = 3; g.items_max = cdiv(R, 128);
      g.k_split = choose_ksplit((long)g.items_max * cdiv(D, g.tile_cols), H * hd, kMaxDenseSplit, &g.k_chunk);
      opp.n = g.k_split;
      g.C = at<float>(ws, p.dpart); g.ldc = D; g.c_kstride = (long)R * D; g.flag = ps.flag;
      g.waves8 = R >= kWaves8MinRows;
      ProfScope ps_(m, DG_PROF_DENSE, st);
      DG_CK(gemm(EPI_STORE_F32, g, st));
    }
    {
      ProfScope ps_(m, DG_PROF_OTHER, st);
      DG_CK(rmsnorm_rows(h, lw(m, l, m->lay.ffn_norm), R, D, d.rms_eps, xn2, xr, nullptr, opp, nullptr, ps.flag,
                         st));
    }
    // shared FFN: independent of the routed path, so it runs
    // on the side stream, forked here and joined before the combine.  Its
    // kernels are enqueued after the router's: a captured graph then keeps the
    // routed path (the critical one) on the main queue, and only the shared
    // FFN pays the cross-queue latency of the fork; at the join its result is
    // long done.
    Partials ysp{ys, 0, (long)R * D};
    bool forked = false;
    hipStream_t ss = st;
    if (fs && !ns && side_stream(m)) {
      DG_CK(hipEventRecord(m->ev_fork, st));
      ss = m->side;
      forked = true;
    }
    auto shared_ffn = [&]() -> dg_status {
      if (forked) DG_CK(hipStreamWaitEvent(m->side, m->ev_fork, 0));
      ProfScope ps_(m, DG_PROF_SHARED, ss);
      GemmArgs g = gargs();
      g.ring = m->d_ring;
      g.A = xn2; g.lda = D; g.W = lw(m, l, m->lay.w_gate_sh); g.W2 = lw(m, l, m->lay.w_up_sh); g.ldw = D;
      g.K = D; g.N = fs; g.k_chunk = D; dense_rows(g, R); g.C = hs; g.ldc = fs; g.flag = ps.flag;
      DG_CK(gemm(EPI_GEGLU_BF16, g, ss));
      GemmArgs g2 = gargs();
      g2.ring = m->d_ring;
      g2.A = hs; g2.lda = fs; g2.W = lw(m, l, m->lay.w_down_sh); g2.ldw = fs; g2.K = fs; g2.N = D;
      g2.C = ys; g2.ldc = D; g2.c_kstride = (long)R * D; g2.flag = ps.flag;
      if (forked && fat_rows(R) && gemm_fat_pitch_ok(fs, fs)) {
        // beside the expert products, a few long workgroups (256 x 128 output
        // tiles, no k split: 22 at 256 rows) hold fewer of the slots those
        // products could fill than hundreds of short split-K ones; the join is
        // far off, so their length costs nothing (full step 9.29 -> 9.16 ms)
        g2.M = R; g2.items_max = cdiv(R, kFatRowChunk); g2.k_split = 1; g2.k_chunk = fs;
        ysp.n = 1;
        DG_CK(gemm_fat(EPI_STORE_F32, g2, ss));
      } else {
        dense_rows(g2, R);
        g2.tile_rows = 128; g2.ring = 3; g2.items_max = cdiv(R, 128);   // as the O projection
        g2.k_split = choose_ksplit((long)g2.items_max * cdiv(D, g2.tile_cols), fs, kMaxDenseSplit, &g2.k_chunk);
        ysp.n = g2.k_split;
        g2.waves8 = R >= kWaves8MinRows;
        DG_CK(gemm(EPI_STORE_F32, g2, ss));
      }
      if (forked) DG_CK(hipEventRecord(m->ev_join, ss));
      return DG_OK;
    };
    // router logits (hi and lo rows, split-K partials) and top-k
    Partials rlp{rlog, 1, (long)2 * R * E};
    {
      GemmArgs g = gargs();
      g.ring = m->d_ring;
      g.A = xr; g.lda = D; g.W = lw(m, l, m->lay.w_router); g.ldw = D; g.K = D; g.N = E;
      dense_rows(g, 2 * R);
      g.k_split = choose_ksplit((long)g.items_max * cdiv(E, 64), D, kMaxRouterSplit, &g.k_chunk);
      rlp.n = g.k_split;
      g.C = rlog; g.ldc = E; g.c_kstride = (long)2 * R * E; g.flag = ps.flag;
      g.waves8 = 2 * R >= kWaves8MinRows;
      ProfScope ps_(m, DG_PROF_ROUTER, st);
      DG_CK(gemm(EPI_STORE_F32, g, st));
    }
    {
      ProfScope psr_(m, DG_PROF_ROUTER, st);
      int32_t* edump = ps.expert_dump ? ps.expert_dump + (size_t)l * R * k : nullptr;
      float* gdump = ps.gate_dump ? ps.gate_dump + (size_t)l * R * k : nullptr;
      float* rdump = ps.router_dump ? ps.router_dump + (size_t)l * R * E : nullptr;
      if (R <= 4) {   // decoding: one launch
        DG_CK(router_topk_permute(rlp, R, E, k, ns, eidx, egate, edump, gdump, rdump, cnt, off, slot_of, slot_row, items,
                                  nitems, m->x_rows, ps.flag, st));
      } else {
        DG_CK(router_topk(rlp, R, E, k, ns, eidx, egate, edump, gdump, rdump, ps.flag, st));
        DG_CK(moe_permute(eidx, R, kx, Ex, cnt, off, slot_of, slot_row, items, nitems, m->x_rows, ps.flag, st));
      }
    }
    if (fs && !ns) {
      dg_status sr = shared_ffn();
      if (sr != DG_OK) return sr;
    }
    // experts: gate/up (GEGLU) then down, grouped by expert over the permuted slots
    {
      GemmArgs g = gargs();
      g.A = xn2; g.lda = D; g.a_rows = slot_row; g.W = lw(m, l, m->lay.w_gate); g.W2 = lw(m, l, m->lay.w_up);
      g.ldw = D; g.w_gstride = (long)fe * D; g.K = D; g.N = fe; g.k_chunk = D;
      g.items = items; g.n_items = nitems; g.items_max = items_max; g.tile_rows = m->x_rows; g.tile_cols = m->x_cols; g.ring = m->x_ring;
      g.few_rows = R <= kGemvRows ? R : 0;   // an expert takes each row at most once
      if (ns) {   // shared gate / up blocks [ns][fe][D]
        g.Wx = lw(m, l, m->lay.w_gate_sh); g.Wx2 = lw(m, l, m->lay.w_up_sh); g.ldwx = D;
        g.wx_gstride = (long)fe * D; g.grp_x = E;
      }
      g.C = hbuf; g.ldc = fe; g.flag = ps.flag;
      ProfScope ps_(m, DG_PROF_EXPERT_GATEUP, st);
      DG_CK(gemm(EPI_GEGLU_BF16, g, st));
    }
    {
      GemmArgs g = gargs();
      g.A = hbuf; g.lda = fe; g.W = lw(m, l, m->lay.w_down); g.ldw = fe; g.w_gstride = (long)D * fe; g.K = fe;
      g.N = D; g.k_chunk = fe; g.items = items; g.n_items = nitems; g.items_max = items_max;
      g.tile_rows = m->x_rows; g.tile_cols = m->xd_cols; g.ring = m->xd_ring;
      g.few_rows = R <= kGemvRows ? R : 0;
      if (ns) {   // shared down block c: columns c fe .. of [D][fs]
        g.Wx = lw(m, l, m->lay.w_down_sh); g.ldwx = fs; g.wx_gstride = fe; g.grp_x = E;
      }
      g.C = ybuf; g.ldc = D; g.flag = ps.flag;
      ProfScope ps_(m, DG_PROF_EXPERT_DOWN, st);
      DG_CK(gemm(EPI_STORE_BF16, g, st));
    }
    if (forked) DG_CK(hipStreamWaitEvent(st, m->ev_join, 0));
    const bf16_t* nw = nullptr;
    if (l + 1 < d.n_layers) nw = lw(m, l + 1, m->lay.attn_norm);
    else if (ps.final_norm) nw = (const bf16_t*)m->w.final_norm;
    {
      ProfScope psc_(m, DG_PROF_OTHER, st);
      DG_CK(moe_combine(h, ysp, ybuf, slot_of, egate, R, D, kx, nw, d.rms_eps, xn,
                        ps.hidden_dump ? ps.hidden_dump + (size_t)(l + 1) * R * D : nullptr, ps.flag, st));
    }
  }
  return DG_OK;
}

// ---------------------------------------------------------------------------
static dg_status check_step_shapes(const dg_model* m, int Bp, int P, int P_max, int B, int T) {
  if (!m) return DG_ERR_ARG;
  if (B < 1 || T < 1 || P < 0 || P_max < P || Bp < 1) return DG_ERR_ARG;
  if (Bp != 1 && Bp != B) return DG_ERR_ARG;
  if (T % 32 || T > 1024 || P % 32 || P_max % 32 || B > 16) return DG_ERR_SHAPE;
  return DG_OK;
}

extern "C" dg_status dg_forward_hidden(dg_model* m, const void* kv, int32_t Bp, int32_t P, int32_t P_max,
                                       int32_t B, int32_t T, float* hidden, float* hidden_dump,
                                       int32_t* expert_dump, float* gate_dump, void* ws, size_t ws_bytes,
                                       dg_stream_t stream) {
  dg_status s = check_step_shapes(m, Bp, P, P_max, B, T);
  if (s != DG_OK) return s;
  if (!hidden || !ws || (P > 0 && !kv)) return DG_ERR_ARG;
  const int R = B * T;
  const Plan p = make_plan(m->d, R, P + T);
  if (ws_bytes < p.total) return DG_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  // the caller's hidden buffer is the residual stream
  DG_CK(hipMemcpyAsync(at<float>(ws, p.h), hidden, (size_t)R * m->d.d_model * 4, hipMemcpyDeviceToDevice, st));
  DG_CK(rmsnorm_rows(at<float>(ws, p.h), m->layers[0] + m->lay.attn_norm, R, m->d.d_model, m->d.rms_eps,
                     at<bf16_t>(ws, p.xn), nullptr, hidden_dump, Partials{nullptr, 0, 0}, nullptr, nullptr, st));
  Pass ps{};
  ps.rows = R; ps.B = B; ps.per_batch = T; ps.pos0 = P; ps.prefill = false;
  ps.kv = (const bf16_t*)kv; ps.kv_Bp = Bp; ps.Bp = Bp; ps.P = P; ps.P_max = P_max;
  ps.hidden_dump = hidden_dump; ps.expert_dump = expert_dump; ps.gate_dump = gate_dump;
  ps.final_norm = false; ps.flag = nullptr;
  s = run_layers(m, p, ws, ps, st);
  if (s != DG_OK) return s;
  DG_CK(hipMemcpyAsync(hidden, at<float>(ws, p.h), (size_t)R * m->d.d_model * 4, hipMemcpyDeviceToDevice, st));
  return DG_OK;
}

// Optional records of one pass of a prefill (prompt 0, positions pos ..
// pos + n - 1): layer inputs, final hidden, routing.
struct PrefillDump {
  int pos = 0, n = 0;
  float* hidden = nullptr;
  int32_t* experts = nullptr;
  float* gates = nullptr;
  float* router = nullptr;
};

// causal encoding of positions P0 .. P0+n-1 of each of Bp prompts (inputs
// [Bp][n]), against the cached K/V of positions 0 .. P0-1
static dg_status prefill_impl(dg_model* m, const int32_t* tokens, const float* hidden, int Bp, int P0, int n,
                              int P_max, void* kv, void* ws, size_t ws_bytes, hipStream_t st,
                              const PrefillDump& dump = PrefillDump()) {
  if (!m || !kv || !ws || (!tokens && !hidden)) return DG_ERR_ARG;
  if (Bp < 1 || n < 1 || P0 < 0 || P_max < P0 + n) return DG_ERR_ARG;
  if (P_max % 32) return DG_ERR_SHAPE;
  if (tokens && m->d.vocab == 0) return DG_ERR_ARG;
  if (dump.n && (dump.n < 1 || dump.pos < P0 || dump.pos + dump.n > P0 + n)) return DG_ERR_ARG;
  const int P = P0 + n;
  // largest chunk whose workspace fits: all n rows (at most 4096), else a multiple of 32
  int chunk = 0;
  for (int c = std::min(n, 4096); c >= 1; c = c > 32 ? (c - 1) / 32 * 32 : 0)
    if (make_plan(m->d, c, P).total <= ws_bytes) { chunk = c; break; }
  if (chunk == 0) return DG_ERR_WORKSPACE;
  if (dump.n > chunk) return DG_ERR_WORKSPACE;   // the recorded positions make one pass
  const Plan p = make_plan(m->d, chunk, P);
  const dg_model_desc& d = m->d;
  for (int bp = 0; bp < Bp; ++bp) {
    // passes of at most `chunk` rows; with a record, its positions are one pass
    const bool rec = bp == 0 && dump.n > 0;
    for (int q0 = P0; q0 < P;) {
      int R = std::min(chunk, P - q0);
      bool here = false;
      if (rec) {
        if (q0 == dump.pos) {
          R = dump.n;
          here = true;
        } else if (q0 < dump.pos) {
          R = std::min(R, dump.pos - q0);
        }
      }
      if (tokens) {
        DG_CK(embed_rows(tokens + (size_t)bp * n + (q0 - P0), (const bf16_t*)m->w.embed, R, d.d_model,
                         at<float>(ws, p.h), nullptr, st));
      } else {
        DG_CK(hipMemcpyAsync(at<float>(ws, p.h), hidden + ((size_t)bp * n + (q0 - P0)) * d.d_model,
                             (size_t)R * d.d_model * 4, hipMemcpyDeviceToDevice, st));
      }
      DG_CK(rmsnorm_rows(at<float>(ws, p.h), m->layers[0] + m->lay.attn_norm, R, d.d_model, d.rms_eps,
                         at<bf16_t>(ws, p.xn), nullptr, here ? dump.hidden : nullptr, Partials{nullptr, 0, 0},
                         nullptr, nullptr, st));
      Pass ps{};
      ps.rows = R; ps.B = 1; ps.per_batch = R; ps.pos0 = q0; ps.prefill = true; ps.bp = bp; ps.q0 = q0;
      ps.kv = (const bf16_t*)kv; ps.kv_Bp = Bp; ps.Bp = 1; ps.P = 0; ps.P_max = P_max;
      ps.final_norm = false; ps.flag = nullptr;
      if (here) {
        ps.hidden_dump = dump.hidden; ps.expert_dump = dump.experts; ps.gate_dump = dump.gates;
        ps.router_dump = dump.router;
      }
      dg_status s = run_layers(m, p, ws, ps, st);
      if (s != DG_OK) return s;
      q0 += R;
    }
  }
  return DG_OK;
}

extern "C" dg_status dg_prefill_dump(dg_model* m, const int32_t* tokens, int32_t Bp, int32_t P0, int32_t n,
                                     int32_t P_max, void* kv, int32_t dump_pos, int32_t dump_n, float* hidden_dump,
                                     int32_t* expert_dump, float* gate_dump, float* router_dump, void* ws,
                                     size_t ws_bytes, dg_stream_t stream) {
  if (!tokens || dump_n < 1) return DG_ERR_ARG;
  PrefillDump dmp;
  dmp.pos = dump_pos; dmp.n = dump_n; dmp.hidden = hidden_dump; dmp.experts = expert_dump; dmp.gates = gate_dump;
  dmp.router = router_dump;
  return prefill_impl(m, tokens, nullptr, Bp, P0, n, P_max, kv, ws, ws_bytes, (hipStream_t)stream, dmp);
}

extern "C" dg_status dg_prefill_prefix(dg_model* m, const int32_t* prefix, int32_t Bp, int32_t P, int32_t P_max,
                                       void* kv, void* ws, size_t ws_bytes, dg_stream_t stream) {
  if (!prefix) return DG_ERR_ARG;
  if (P % 32) return DG_ERR_SHAPE;
  return prefill_impl(m, prefix, nullptr, Bp, 0, P, P_max, kv, ws, ws_bytes, (hipStream_t)stream);
}

extern "C" dg_status dg_prefill_append(dg_model* m, const int32_t* tokens, int32_t Bp, int32_t P0, int32_t n,
                                       int32_t P_max, void* kv, void* ws, size_t ws_bytes, dg_stream_t stream) {
  if (!tokens) return DG_ERR_ARG;
  return prefill_impl(m, tokens, nullptr, Bp, P0, n, P_max, kv, ws, ws_bytes, (hipStream_t)stream);
}

extern "C" dg_status dg_prefill_hidden(dg_model* m, const float* prefix_hidden, int32_t Bp, int32_t P,
                                       int32_t P_max, void* kv, void* ws, size_t ws_bytes, dg_stream_t stream) {
  if (!prefix_hidden) return DG_ERR_ARG;
  if (P % 32) return DG_ERR_SHAPE;
  return prefill_impl(m, nullptr, prefix_hidden, Bp, 0, P, P_max, kv, ws, ws_bytes, (hipStream_t)stream);
}

// Replay the graph cached under `key`, or capture `enqueue` on `st` into one,
// cache it (up to 8, least recently used evicted) and launch it.
template <class F>
static dg_status graph_run(dg_model* m, const GraphKey& key, F&& enqueue, hipStream_t st) {
  for (GraphEntry& g : m->graphs) {
    if (memcmp(&g.key, &key, sizeof(key)) == 0) {
      g.last_use = ++m->use_clock;
      DG_CK(hipGraphLaunch(g.exec, st));
      return DG_OK;
    }
  }
  DG_CK(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
  dg_status r = enqueue();
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(st, &graph);
  if (r != DG_OK || ec != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    if (r != DG_OK) return r;
    fprintf(stderr, "libdg: stream capture failed: %s\n", hipGetErrorString(ec));
    return DG_ERR_HIP;
  }
  hipGraphExec_t exec = nullptr;
  const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (ei != hipSuccess) {
    fprintf(stderr, "libdg: graph instantiation failed: %s\n", hipGetErrorString(ei));
    return DG_ERR_HIP;
  }
  if (m->graphs.size() >= 8) {
    size_t oldest = 0;
    for (size_t i = 1; i < m->graphs.size(); ++i)
      if (m->graphs[i].last_use < m->graphs[oldest].last_use) oldest = i;
    (void)hipGraphExecDestroy(m->graphs[oldest].exec);
    m->graphs.erase(m->graphs.begin() + oldest);
  }
  m->graphs.push_back(GraphEntry{key, exec, ++m->use_clock});
  DG_CK(hipGraphLaunch(exec, st));
  return DG_OK;
}

// One autoregressive step per sequence: the token at position P is encoded
// against the cached positions 0..P-1 (its K/V written at P), then the final
// norm, the LM head and the next-token sample.  Sequences run one after
// another, each a one-row pass over the layers.  pos_dev: the position is read
// on the device (the P-dependent kernel arguments are then unused), so that
// one captured graph serves every position.
static dg_status ar_impl(dg_model* m, void* kv, int B, int P, int P_max, const int32_t* token, float inv_tau,
                         const uint64_t* row_seeds, int32_t* next, int32_t* argmax, float* entropy,
                         float* logits_dump, void* ws, const Plan& p, const int32_t* pos_dev, hipStream_t st) {
  const dg_model_desc& d = m->d;
  const int V = d.vocab, D = d.d_model;
  float* h = at<float>(ws, p.h);
  bf16_t* xn = at<bf16_t>(ws, p.xn);
  for (int b = 0; b < B; ++b) {
    DG_CK(embed_rows(token + b, (const bf16_t*)m->w.embed, 1, D, h, nullptr, st));
    DG_CK(rmsnorm_rows(h, m->layers[0] + m->lay.attn_norm, 1, D, d.rms_eps, xn, nullptr, nullptr,
                       Partials{nullptr, 0, 0}, nullptr, nullptr, st));
    Pass ps{};
    ps.rows = 1; ps.B = 1; ps.per_batch = 1; ps.pos0 = P; ps.prefill = true; ps.bp = b; ps.q0 = P;
    ps.kv = (const bf16_t*)kv; ps.kv_Bp = B; ps.Bp = 1; ps.P = 0; ps.P_max = P_max;
    ps.final_norm = true; ps.flag = nullptr; ps.pos_dev = pos_dev;
    dg_status s = run_layers(m, p, ws, ps, st);
    if (s != DG_OK) return s;
    float* logits = logits_dump ? logits_dump + (size_t)b * V : at<float>(ws, p.logits);
    {
      GemmArgs g = gargs();
      g.A = xn; g.lda = D; g.W = (const bf16_t*)m->w.embed; g.ldw = D; g.K = D; g.N = V; g.k_chunk = D;
      g.C = logits; g.ldc = V;
      ProfScope ps_(m, DG_PROF_LMHEAD, st);
      DG_CK(dense_gemm(EPI_STORE_F32, g, 1, st));
    }
    ArSampleArgs sa;
    memset(&sa, 0, sizeof(sa));
    sa.logits = logits; sa.B = 1; sa.V = V; sa.ldl = V; sa.inv_tau = inv_tau; sa.pos = P; sa.pos_dev = pos_dev;
    sa.seeds[0] = row_seeds[b]; sa.vsplit = p.vsplit; sa.part = at<float>(ws, p.spart);
    sa.next = next + b; sa.argmax = argmax ? argmax + b : nullptr; sa.entropy = entropy ? entropy + b : nullptr;
    ProfScope ps_(m, DG_PROF_SAMPLER, st);
    DG_CK(ar_sample(sa, st));
  }
  return DG_OK;
}

extern "C" dg_status dg_ar_step(dg_model* m, void* kv, int32_t B, int32_t P, int32_t P_max, const int32_t* token,
                                float tau, const uint64_t* row_seeds, int32_t* next, int32_t* argmax,
                                float* entropy, float* logits_dump, void* ws, size_t ws_bytes,
                                dg_stream_t stream) {
  if (!m || !kv || !token || !next || !row_seeds || !ws) return DG_ERR_ARG;
  if (m->d.vocab == 0) return DG_ERR_UNSUPPORTED;
  if (B < 1 || B > 16 || P < 0 || P_max < P + 1 || !(tau > 0.f) || !std::isfinite(tau)) return DG_ERR_ARG;
  if (P_max % 32 || m->d.vocab % 4) return DG_ERR_SHAPE;
  const Plan p = make_plan(m->d, 1, P + 1);
  if (ws_bytes < p.total) return DG_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const float inv_tau = (float)(1.0 / (double)tau);
  if (!m->use_graphs || m->prof.on || st == nullptr)
    return ar_impl(m, kv, B, P, P_max, token, inv_tau, row_seeds, next, argmax, entropy, logits_dump, ws, p,
                   nullptr, st);
  // graph replay: the position goes to the device first; every other argument
  // is part of the graph's key
  int32_t* pos_dev = at<int32_t>(ws, p.pos);
  DG_CK(fill_i32(pos_dev, P, 1, st));
  GraphKey key;
  memset(&key, 0, sizeof(key));
  key.kind = 2;
  key.kv = kv; key.Bp = B; key.P_max = P_max; key.B = B; key.T = 1;
  key.c.tokens = const_cast<int32_t*>(token); key.c.xhat = next; key.c.argmax = argmax; key.c.entropy = entropy;
  key.c.logits_dump = logits_dump;
  key.tau_start = inv_tau;
  for (int b = 0; b < B; ++b) key.seeds[b] = row_seeds[b];
  key.ws = ws; key.ws_bytes = ws_bytes;
  return graph_run(m, key, [&]() -> dg_status {
    return ar_impl(m, kv, B, P, P_max, token, inv_tau, row_seeds, next, argmax, entropy, logits_dump, ws, p,
                   pos_dev, st);
  }, st);
}

// ---------------------------------------------------------------------------
static dg_status check_sampler(const dg_sampler* sp, int B) {
  if (!sp || !sp->row_seeds) return DG_ERR_ARG;
  if (sp->max_steps < 1 || (sp->lock_rule != 0 && sp->lock_rule != 1) || (sp->stop_rule != 0 && sp->stop_rule != 1))
    return DG_ERR_ARG;
  if (!(sp->tau_start > 0.f) || !(sp->tau_end > 0.f)) return DG_ERR_ARG;
  (void)B;
  return DG_OK;
}

static dg_status check_canvas(const dg_canvas* c, bool need_sc) {
  if (!c || !c->tokens || !c->locked || !c->entropy || !c->xhat || !c->argmax || !c->stopped || !c->steps)
    return DG_ERR_ARG;
  if (need_sc && !c->self_cond) return DG_ERR_ARG;
  return DG_OK;
}

static SampleArgs sample_args(const float* logits, int B, int T, int V, dg_canvas* c, int step_arg,
                              const dg_sampler* sp, float* part, int vsplit, float4* rowstat, int32_t* all_stopped,
                              const int32_t* flag) {
  SampleArgs a;
  memset(&a, 0, sizeof(a));
  a.logits = logits; a.B = B; a.T = T; a.V = V; a.ldl = V; a.step_arg = step_arg;
  a.tau_start = sp->tau_start; a.tau_end = sp->tau_end; a.max_steps = sp->max_steps;
  a.lock_rule = sp->lock_rule; a.lock_thresh = sp->lock_thresh; a.stop_rule = sp->stop_rule;
  a.stop_thresh = sp->stop_thresh;
  for (int b = 0; b < B && b < 16; ++b) a.seeds[b] = sp->row_seeds[b];
  a.vsplit = vsplit; a.part = part; a.rowstat = rowstat;
  a.tokens = c->tokens; a.locked = c->locked; a.entropy = c->entropy; a.xhat = c->xhat; a.argmax = c->argmax;
  a.stopped = c->stopped; a.steps = c->steps; a.all_stopped = all_stopped; a.flag = flag;
  return a;
}

// one full step; step_arg < 0: step index read from canvas->steps on the device
static dg_status step_impl(dg_model* m, const void* kv, int Bp, int P, int P_max, int B, int T, dg_canvas* c,
                           int step_arg, const dg_sampler* sp, void* ws, const Plan& p, const int32_t* flag,
                           int32_t* all_stopped, hipStream_t st) {
  const dg_model_desc& d = m->d;
  const int R = B * T, D = d.d_model, V = d.vocab;
  float* h = at<float>(ws, p.h);
  bf16_t* xn = at<bf16_t>(ws, p.xn);
  DG_CK(embed_rows(c->tokens, (const bf16_t*)m->w.embed, R, D, h, flag, st));
  // self-conditioning: split-K partials of s_prev W_sc^T, gated and added by the first norm
  Partials scp{at<float>(ws, p.dpart), 0, (long)R * D};
  if (d.self_cond) {
    GemmArgs g = gargs();
    g.ring = m->d_ring;
    g.A = (const bf16_t*)c->self_cond; g.lda = D; g.W = (const bf16_t*)m->w.self_cond_w; g.ldw = D; g.K = D;
    g.N = D; dense_rows(g, R);
    if (R >= kWaves8MinRows) {   // as the O projection: 128-row tiles on the 8-wave kernel
      g.tile_rows = 128; g.ring = 3; g.items_max = cdiv(R, 128); g.waves8 = 1;
    }
    g.k_split = choose_ksplit((long)g.items_max * cdiv(D, 64), D, kMaxDenseSplit, &g.k_chunk);
    scp.n = g.k_split;
    g.C = at<float>(ws, p.dpart); g.ldc = D; g.c_kstride = (long)R * D; g.flag = flag;
    ProfScope ps_(m, DG_PROF_DENSE, st);
    DG_CK(gemm(EPI_STORE_F32, g, st));
  }
  DG_CK(rmsnorm_rows(h, m->layers[0] + m->lay.attn_norm, R, D, d.rms_eps, xn, nullptr, c->hidden_dump, scp,
                     (const bf16_t*)m->w.self_cond_gate, flag, st));
  Pass ps{};
  ps.rows = R; ps.B = B; ps.per_batch = T; ps.pos0 = P; ps.prefill = false;
  ps.kv = (const bf16_t*)kv; ps.kv_Bp = Bp; ps.Bp = Bp; ps.P = P; ps.P_max = P_max;
  ps.hidden_dump = c->hidden_dump; ps.expert_dump = c->expert_dump; ps.gate_dump = c->gate_dump;
  ps.router_dump = c->router_dump;
  ps.final_norm = true; ps.flag = flag;
  dg_status s = run_layers(m, p, ws, ps, st);
  if (s != DG_OK) return s;
  // LM head: logits = rms(h) E^T (fp32, 256 x 256 tiles over the vocabulary).
  // The softmax statistics then come per vocabulary slice (the slices of the
  // soft-prediction product's split contraction), merged per row online: the
  // entropy and argmax for the sampler, and the slice weights of s_next.  The
  // Gumbel-max pass over the logits (Philox-bound ALU work) runs on the side
  // stream beside the memory-bound slice statistics; the finishing pass joins
  // both.  (Beside the soft-prediction product instead, it keeps that
  // product's one-workgroup-per-CU tiles off the CUs it occupies: slower.)
  float* logits = c->logits_dump ? c->logits_dump : at<float>(ws, p.logits);
  {
    GemmArgs g = gargs();
    g.A = xn; g.lda = D; g.W = (const bf16_t*)m->w.embed; g.ldw = D; g.K = D; g.N = V; g.k_chunk = D;
    g.C = logits; g.ldc = V; g.flag = flag;
    ProfScope ps_(m, DG_PROF_LMHEAD, st);
    DG_CK(dense_gemm(EPI_STORE_F32, g, R, st));
  }
  float4* rowstat = at<float4>(ws, p.rowstat);
  float4* sstat = at<float4>(ws, p.sstat);
  SampleArgs sa = sample_args(logits, B, T, V, c, step_arg, sp, at<float>(ws, p.spart), p.vsplit, nullptr,
                              nullptr, flag);
  sa.rowstat_in = rowstat;
  bool forked = false;
  if (side_stream(m)) {
    DG_CK(hipEventRecord(m->ev_fork, st));
    DG_CK(hipStreamWaitEvent(m->side, m->ev_fork, 0));
    {
      ProfScope ps_(m, DG_PROF_SAMPLER, m->side);
      DG_CK(sample_partial(sa, m->side));
    }
    DG_CK(hipEventRecord(m->ev_join, m->side));
    forked = true;
  }
  {
    ProfScope ps_(m, d.self_cond ? DG_PROF_SOFTEMB : DG_PROF_SAMPLER, st);
    bf16_t* P_ = d.self_cond ? at<bf16_t>(ws, p.P) : nullptr;
    DG_CK(softmax_slices(logits, V, R, V, p.kchunk, p.ksplit, T, c->stopped, P_, sstat, flag, st));
    float* part = nullptr;
    if (d.self_cond) {
      // s_next partials per vocabulary slice: P~ [R][V] times E [V][d] as stored
      GemmArgs g = gargs();
      g.A = P_; g.lda = V; g.W = (const bf16_t*)m->w.embed; g.ldw = D; g.K = V; g.N = D; g.k_chunk = p.kchunk;
      g.k_split = p.ksplit; g.C = at<float>(ws, p.separt); g.ldc = D;
      g.c_kstride = (long)R * D; g.flag = flag; g.M = R; g.items_max = cdiv(R, 256);
      DG_CK(gemm_kn(g, st));
      part = at<float>(ws, p.separt);
    }
    DG_CK(softmax_finish(sstat, p.ksplit, R, T, c->stopped, part, D, (bf16_t*)c->self_cond, rowstat, flag, st));
  }
  if (forked) DG_CK(hipStreamWaitEvent(st, m->ev_join, 0));
  {
    ProfScope ps_(m, DG_PROF_SAMPLER, st);
    if (!forked) DG_CK(sample_partial(sa, st));
    DG_CK(sample_finish(sa, st));
  }
  (void)all_stopped;
  return DG_OK;
}

__global__ void dg_all_stopped_kernel(const int32_t* stopped, int B, int32_t* flag) {
  if (threadIdx.x == 0) {
    int all = 1;
    for (int b = 0; b < B; ++b) all &= (stopped[b] != 0);
    *flag = all;
  }
}

// Enqueue one step whose step index is read from canvas->steps on the device,
// as a replay of a captured hipGraph when possible (the default stream cannot
// be captured, and profiling records events: those run the launches directly).
static dg_status step_device_indexed(dg_model* m, const void* kv, int Bp, int P, int P_max, int B, int T,
                                     dg_canvas* c, const dg_sampler* sp, void* ws, size_t ws_bytes, const Plan& p,
                                     int32_t* flag, hipStream_t st) {
  auto enqueue = [&]() -> dg_status {
    dg_status r = step_impl(m, kv, Bp, P, P_max, B, T, c, -1, sp, ws, p, flag, nullptr, st);
    if (r != DG_OK) return r;
    if (flag) {
      hipLaunchKernelGGL(dg_all_stopped_kernel, dim3(1), dim3(64), 0, st, c->stopped, B, flag);
      DG_CK(hipGetLastError());
    }
    return DG_OK;
  };
  if (!m->use_graphs || m->prof.on || st == nullptr) return enqueue();
  GraphKey key;
  memset(&key, 0, sizeof(key));
  key.kind = flag ? 1 : 0;
  key.kv = kv; key.Bp = Bp; key.P = P; key.P_max = P_max; key.B = B; key.T = T;
  key.c = *c;
  key.tau_start = sp->tau_start; key.tau_end = sp->tau_end; key.lock_thresh = sp->lock_thresh;
  key.stop_thresh = sp->stop_thresh; key.max_steps = sp->max_steps; key.lock_rule = sp->lock_rule;
  key.stop_rule = sp->stop_rule;
  for (int b = 0; b < B && b < 16; ++b) key.seeds[b] = sp->row_seeds[b];
  key.ws = ws; key.ws_bytes = ws_bytes;
  return graph_run(m, key, enqueue, st);
}

extern "C" dg_status dg_denoise_step(dg_model* m, const void* kv, int32_t Bp, int32_t P, int32_t P_max, int32_t B,
                                     int32_t T, dg_canvas* canvas, int32_t step, const dg_sampler* sp, void* ws,
                                     size_t ws_bytes, dg_stream_t stream) {
  dg_status s = check_step_shapes(m, Bp, P, P_max, B, T);
  if (s != DG_OK) return s;
  if (m->d.vocab == 0) return DG_ERR_UNSUPPORTED;
  if ((s = check_sampler(sp, B)) != DG_OK) return s;
  if ((s = check_canvas(canvas, m->d.self_cond != 0)) != DG_OK) return s;
  if (step < 0 || !ws || (P > 0 && !kv)) return DG_ERR_ARG;
  const Plan p = make_plan(m->d, B * T, P + T);
  if (ws_bytes < p.total) return DG_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  // the step index of every running row goes to the device; the step itself
  // reads it there, so one captured graph serves every step index
  DG_CK(set_step(canvas->steps, canvas->stopped, B, step, st));
  return step_device_indexed(m, kv, Bp, P, P_max, B, T, canvas, sp, ws, ws_bytes, p, nullptr, st);
}

extern "C" dg_status dg_generate_block(dg_model* m, const void* kv, int32_t Bp, int32_t P, int32_t P_max,
                                       int32_t B, int32_t T, dg_canvas* canvas, const dg_sampler* sp,
                                       int32_t poll_every, void* ws, size_t ws_bytes, dg_stream_t stream) {
  dg_status s = check_step_shapes(m, Bp, P, P_max, B, T);
  if (s != DG_OK) return s;
  if (m->d.vocab == 0) return DG_ERR_UNSUPPORTED;
  if ((s = check_sampler(sp, B)) != DG_OK) return s;
  if ((s = check_canvas(canvas, m->d.self_cond != 0)) != DG_OK) return s;
  if (poll_every < 0 || !ws || (P > 0 && !kv)) return DG_ERR_ARG;
  const Plan p = make_plan(m->d, B * T, P + T);
  if (ws_bytes < p.total) return DG_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  int32_t* flag = at<int32_t>(ws, p.flag);
  DG_CK(fill_i32(flag, 0, 1, st));
  DG_CK(fill_i32(canvas->stopped, 0, B, st));
  DG_CK(fill_i32(canvas->steps, 0, B, st));
  if (m->d.self_cond)
    DG_CK(fill_u16((uint16_t*)canvas->self_cond, 0, (long)B * T * m->d.d_model, st));
  for (int step = 0; step < sp->max_steps; ++step) {
    s = step_device_indexed(m, kv, Bp, P, P_max, B, T, canvas, sp, ws, ws_bytes, p, flag, st);
    if (s != DG_OK) return s;
    if (poll_every > 0 && (step + 1) % poll_every == 0 && step + 1 < sp->max_steps) {
      int32_t hf = 0;
      DG_CK(hipMemcpyAsync(&hf, flag, sizeof(int32_t), hipMemcpyDeviceToHost, st));
      DG_CK(hipStreamSynchronize(st));
      if (hf) break;
    }
  }
  return DG_OK;
}

// ---------------------------------------------------------------------------
extern "C" size_t dg_sample_workspace_bytes(int32_t B, int32_t T, int32_t V) {
  if (B < 1 || T < 1 || V < 1) return 0;
  const int rows = B * T;
  return al256((size_t)rows * vsplit_of(rows, V) * 8 * 4) + al256((size_t)rows * 16);
}

// argument checks of the sampler entry points (no device work)
static dg_status check_sample_args(const float* logits, int B, int T, int V, const dg_canvas* canvas, int step,
                                   const dg_sampler* sp) {
  if (!logits || step < 0) return DG_ERR_ARG;
  if (B < 1 || T < 1 || V < 1) return DG_ERR_ARG;
  if (B > 16 || T % 4 || T > 1024) return DG_ERR_SHAPE;
  dg_status s = check_sampler(sp, B);
  if (s != DG_OK) return s;
  return check_canvas(canvas, false);
}

// the sampler's launches over scratch ws (at least dg_sample_workspace_bytes(B, T, V) bytes)
static dg_status sample_logits_impl(const float* logits, int B, int T, int V, dg_canvas* canvas, int step,
                                    const dg_sampler* sp, void* ws, size_t ws_bytes, hipStream_t st) {
  dg_status s = check_sample_args(logits, B, T, V, canvas, step, sp);
  if (s != DG_OK) return s;
  if (!ws) return DG_ERR_ARG;
  if (ws_bytes < dg_sample_workspace_bytes(B, T, V)) return DG_ERR_WORKSPACE;
  const int rows = B * T;
  const int vs = vsplit_of(rows, V);
  float* part = (float*)ws;
  float4* rowstat = at<float4>(ws, al256((size_t)rows * vs * 8 * 4));
  SampleArgs sa = sample_args(logits, B, T, V, canvas, step, sp, part, vs, rowstat, nullptr, nullptr);
  DG_CK(sample_partial(sa, st));
  DG_CK(sample_finish(sa, st));
  return DG_OK;
}

extern "C" dg_status dg_sample_logits(const float* logits, int32_t B, int32_t T, int32_t V, dg_canvas* canvas,
                                      int32_t step, const dg_sampler* sp, void* ws, size_t ws_bytes,
                                      dg_stream_t stream) {
  return sample_logits_impl(logits, B, T, V, canvas, step, sp, ws, ws_bytes, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// dg_sample_logits_noalloc: the sampler over a scratch area that the library
// owns, for callers that cannot allocate.  The area is a file-scope device
// array (one copy per GPU, held until the process ends).  In host code its
// name stands for no device address: the address is fetched once per device
// with hipGetSymbolAddress and only that address is handed to kernels.
// The largest request the sampler accepts (B 16, T 1024) needs 768 KB.
static constexpr size_t kSampleScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) unsigned char scratch[kSampleScratchBytes];
static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// the scratch array's address on the current device (looked up on first use)
static dg_status scratch_on_current_device(void** out) {
  int dev = -1;
  DG_CK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return DG_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    DG_CK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return DG_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DG_OK;
}

extern "C" size_t dg_sample_noalloc_max_bytes(void) { return kSampleScratchBytes; }

extern "C" dg_status dg_sample_logits_noalloc(const float* logits, int32_t B, int32_t T, int32_t V,
                                              dg_canvas* canvas, int32_t step, const dg_sampler* sp,
                                              dg_stream_t stream) {
  dg_status s = check_sample_args(logits, B, T, V, canvas, step, sp);
  if (s != DG_OK) return s;
  if (dg_sample_workspace_bytes(B, T, V) > kSampleScratchBytes) return DG_ERR_WORKSPACE;
  void* ws = nullptr;
  s = scratch_on_current_device(&ws);
  if (s != DG_OK) return s;
  return sample_logits_impl(logits, B, T, V, canvas, step, sp, ws, kSampleScratchBytes, (hipStream_t)stream);
}

extern "C" dg_status dg_init_canvas(const dg_model* m, dg_canvas* c, int32_t B, int32_t T,
                                    const uint64_t* row_seeds, dg_stream_t stream) {
  if (!m || !c || !c->tokens || !c->stopped || !c->steps || !c->argmax || !row_seeds) return DG_ERR_ARG;
  if (B < 1 || T < 1) return DG_ERR_ARG;
  if (B > 16) return DG_ERR_SHAPE;
  if (m->d.vocab == 0) return DG_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  DG_CK(init_canvas(c->tokens, B, T, m->d.vocab, row_seeds, st));
  DG_CK(fill_i32(c->stopped, 0, B, st));
  DG_CK(fill_i32(c->steps, 0, B, st));
  DG_CK(fill_i32(c->argmax, 0, (long)B * T, st));
  if (c->self_cond) DG_CK(fill_u16((uint16_t*)c->self_cond, 0, (long)B * T * m->d.d_model, st));
  return DG_OK;
}

extern "C" dg_status dg_gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, int32_t M, int32_t N,
                                  int32_t K, float* Cm, int64_t ldc, dg_stream_t stream) {
  if (!A || !W || !Cm || M < 1 || N < 1 || K < 1 || lda < K || ldw < K || ldc < N) return DG_ERR_ARG;
  if (K % 64 || lda % 8 || ldw % 8) return DG_ERR_SHAPE;
  GemmArgs g = gargs();
  g.A = (const bf16_t*)A; g.lda = lda; g.W = (const bf16_t*)W; g.ldw = ldw; g.K = K; g.N = N; g.k_chunk = K;
  g.C = Cm; g.ldc = ldc;
  DG_CK(dense_gemm(EPI_STORE_F32, g, M, (hipStream_t)stream));
  return DG_OK;
}

extern "C" dg_status dg_gemm_bf16_kn(const void* A, int64_t lda, const void* W, int64_t ldw, int32_t M, int32_t N,
                                     int32_t K, float* Cm, int64_t ldc, dg_stream_t stream) {
  if (!A || !W || !Cm || M < 1 || N < 1 || K < 1 || lda < K || ldw < N || ldc < N) return DG_ERR_ARG;
  if (K % 64 || N % 8 || lda % 8 || ldw % 8) return DG_ERR_SHAPE;
  if (256L * lda * 2 >= 0x7FFFFFFFL || (64L * ldw + N) * 2 >= 0x7FFFFFFFL) return DG_ERR_SHAPE;
  GemmArgs g = gargs();
  g.A = (const bf16_t*)A; g.lda = lda; g.W = (const bf16_t*)W; g.ldw = ldw; g.K = K; g.N = N; g.k_chunk = K;
  g.C = Cm; g.ldc = ldc; g.M = M; g.items_max = cdiv(M, 256);
  DG_CK(gemm_kn(g, (hipStream_t)stream));
  return DG_OK;
}

// host-side reference entry points of the sampler arithmetic
extern "C" void dg_host_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const dg_u32x4 r = dg_philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1]);
  for (int i = 0; i < 4; ++i) out[i] = r.x[i];
}
extern "C" float dg_host_ln(float x) { return dg_ln(x); }
extern "C" float dg_host_gumbel_of_word(uint32_t w) { return dg_gumbel(dg_uniform_open01(w)); }
extern "C" float dg_host_inv_tau(float t0, float t1, int32_t S, int32_t s) { return dg_inv_tau(t0, t1, S, s); }
extern "C" void dg_host_ln_batch(const float* x, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = dg_ln(x[i]);
}
extern "C" void dg_host_gumbel_batch(const uint32_t* w, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = dg_gumbel(dg_uniform_open01(w[i]));
}

extern "C" dg_status dg_profile_enable(dg_model* m, int32_t on) {
  if (!m) return DG_ERR_ARG;
  m->prof.on = on != 0;
  m->prof.used = 0;
  return DG_OK;
}

extern "C" dg_status dg_profile_read(dg_model* m, int32_t cls, double* total_ms, int32_t* count) {
  if (!m || !total_ms || !count || cls < 0 || cls >= DG_PROF_NCLASS) return DG_ERR_ARG;
  double t = 0.0;
  int n = 0;
  for (size_t i = 0; i < m->prof.used; ++i) {
    if (m->prof.cls[i] != cls) continue;
    DG_CK(hipEventSynchronize(m->prof.pool[2 * i + 1]));
    float ms = 0.f;
    DG_CK(hipEventElapsedTime(&ms, m->prof.pool[2 * i], m->prof.pool[2 * i + 1]));
    t += ms;
    ++n;
  }
  *total_ms = t;
  *count = n;
  return DG_OK;
}
