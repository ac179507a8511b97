/* libdg — one denoising step of a discrete-diffusion mixture-of-experts LM on
 * AMD MI355X (gfx950), behind a plain C ABI.
 *
 * The method (DiffusionGemma technical report: arXiv abstract page at 66bd.net
 * and the chatpaper.ai English abstract; the laozijiushiniubi.cn article,
 * sections 1, 2, 4 and 5; the gxsgwd.com news item):
 *   - the prompt is encoded once with causal attention; its key/value cache is
 *     read by every refinement step of a 256-token block (article section 5);
 *   - a canvas of 256 tokens, initially uniform random vocabulary tokens, is
 *     refined in parallel: each step is one forward pass with bidirectional
 *     attention inside the canvas over the cached prefix (section 2), through
 *     mixture-of-experts layers with 128 experts of which 8 are used per token,
 *     plus a self-conditioning input built from the previous step's prediction;
 *   - the sampler computes a per-position entropy, keeps confident positions
 *     and re-randomises the others with uniform vocabulary noise; locked tokens
 *     can still change later (sections 1 and 4); the temperature anneals
 *     linearly from 0.8 to 0.4; generation stops adaptively on low mean
 *     entropy or at 48 steps (section 4).
 *
 * Conventions (all calls):
 *   - Device pointers point to memory the caller owns (weights, KV cache,
 *     canvas state, workspace).  The library allocates no device memory; it
 *     keeps host-side bookkeeping only (and, for dg_sample_logits_noalloc
 *     alone, one static device array of 1 MiB).
 *   - Calls are stream-ordered and asynchronous: they enqueue kernels on
 *     `stream` and return.  Results are valid after the caller synchronises.
 *   - Arguments are checked before anything is enqueued; on a negative status
 *     nothing has been enqueued.  HIP launch errors return DG_ERR_HIP.
 *   - A dg_model may be used from one stream at a time.
 *   - bf16 tensors are raw 16-bit bfloat16 patterns, row-major.
 *   - Restrictions of this implementation: head_dim in {64, 128, 256};
 *     n_heads / n_kv_heads in {1, 2, 4}; d_model, d_expert, d_shared and
 *     n_heads*head_dim multiples of 64 and d_model <= 4096; n_experts <= 255;
 *     top_k in {1, 2, 4, 8}; canvas length T a multiple of 32 and <= 1024; prefix
 *     lengths P of a prefill or denoising step and capacities P_max multiples of
 *     32 (dg_prefill_append and dg_ar_step start at any position); batch B <= 16;
 *     vocab a multiple of 128.
 *   - Cache positions not yet written must hold finite values (zero the cache
 *     once when allocating it): a pass that ends inside a 32-key tile reads the
 *     whole tile and masks the unwritten keys.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dg_stream_t; /* a hipStream_t */

typedef enum {
  DG_OK = 0,
  DG_ERR_ARG = -1,         /* null pointer or invalid scalar argument            */
  DG_ERR_SHAPE = -2,       /* shape outside the supported set (see above)       */
  DG_ERR_WORKSPACE = -3,   /* ws_bytes smaller than dg_workspace_bytes(...)      */
  DG_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed         */
  DG_ERR_UNSUPPORTED = -5  /* valid request this build does not implement       */
} dg_status;

/* Shapes of the transformer.  vocab == 0 describes a stack of layers without
 * embedding or LM head (hidden states in, hidden states out).  d_shared == 0:
 * no shared FFN.  self_cond: 1 adds h += sigmoid(g) * (s_prev W_sc^T) to the
 * canvas input, s_prev being the previous step's soft-prediction embedding
 * sum_v softmax(logits)_v E_v (article section 2: self-conditioning). */
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, d_expert, d_shared, vocab, self_cond;
  float rope_theta, rms_eps;
} dg_model_desc;

/* Element offsets (bf16 elements) of each tensor inside one packed layer block.
 * Matrices are [out_features][in_features]:
 *   attn_norm [d]; w_qkv [(H + 2 Hkv) hd][d] (q heads, then k heads, then v heads);
 *   q_norm [hd]; k_norm [hd]; w_o [d][H hd]; ffn_norm [d]; w_router [E][d];
 *   w_gate, w_up [E][d_expert][d]; w_down [E][d][d_expert];
 *   w_gate_sh, w_up_sh [d_shared][d]; w_down_sh [d][d_shared].
 * Each offset is a multiple of 128 elements (256 bytes). */
typedef struct {
  size_t attn_norm, w_qkv, q_norm, k_norm, w_o, ffn_norm, w_router;
  size_t w_gate, w_up, w_down, w_gate_sh, w_up_sh, w_down_sh;
  size_t total;
} dg_layer_layout;

/* Device weights (bf16).  embed [vocab][d] is the tied input embedding, the
 * LM head and (read as stored, contracting over the vocabulary) the matrix of
 * the soft-prediction embedding; final_norm [d]; self_cond_w [d][d];
 * self_cond_gate [d].  layers is a HOST array of n_layers device pointers,
 * each to a block laid out as dg_layer_layout.  The pointers are borrowed
 * until dg_model_destroy. */
typedef struct {
  const void* embed;
  const void* final_norm;
  const void* self_cond_w;
  const void* self_cond_gate;
  const void* const* layers;
} dg_weights;

/* Sampler parameters (article section 4).  Temperature of step s:
 * tau = tau_start + (tau_end - tau_start) * s / (max_steps - 1), in fp64.
 * lock_rule 0: position i locks if H_i < lock_thresh; 1: positions sorted by
 * (H_i, i) lock while the running sum of H stays <= lock_thresh.
 * stop_rule 0: stop when mean H < stop_thresh; 1: additionally the argmax of
 * every position equals the previous step's.  Always stop at max_steps.
 * row_seeds: HOST array [B] of 64-bit Philox keys (low word = key word 0). */
typedef struct {
  float tau_start, tau_end;
  int32_t max_steps;
  int32_t lock_rule;
  float lock_thresh;
  int32_t stop_rule;
  float stop_thresh;
  const uint64_t* row_seeds;
} dg_sampler;

/* Canvas state, device pointers, rows b = 0..B-1 of T positions each.
 *   tokens    int32 [B][T] in/out: current canvas, replaced by the next one
 *   locked    uint8 [B][T] out: lock decision of the last step
 *   entropy   fp32  [B][T] out: per-position entropy (nats, temperature 1)
 *   xhat      int32 [B][T] out: the step's Gumbel-max sample
 *   argmax    int32 [B][T] in/out: argmax of the logits (previous one is read
 *                          by stop_rule 1)
 *   self_cond bf16  [B][T][d] in/out: s_prev in, s_next out (zero at step 0);
 *                          may be NULL when self_cond == 0
 *   stopped   int32 [B] in/out; steps int32 [B] in/out (steps taken)
 * Optional outputs (NULL to skip; for parity checks):
 *   logits_dump  fp32 [B][T][vocab]
 *   hidden_dump  fp32 [n_layers + 1][B*T][d]: input of every layer, then the
 *                final hidden state (before the final norm)
 *   expert_dump  int32 [n_layers][B*T][top_k]; gate_dump fp32 same shape
 *   router_dump  fp32 [n_layers][B*T][n_experts]: the router logits the top-k
 *                chose from
 * A stopped row (stopped[b] != 0 on entry) is left unchanged. */
typedef struct {
  int32_t* tokens;
  uint8_t* locked;
  float* entropy;
  int32_t* xhat;
  int32_t* argmax;
  void* self_cond;
  int32_t* stopped;
  int32_t* steps;
  float* logits_dump;
  float* hidden_dump;
  int32_t* expert_dump;
  float* gate_dump;
  float* router_dump;
} dg_canvas;

typedef struct dg_model dg_model;

const char* dg_status_string(dg_status s);

/* Offsets of one packed layer block for `desc`. */
dg_status dg_layer_layout_get(const dg_model_desc* desc, dg_layer_layout* out);

/* Validate shapes and record the weight pointers.  No device work. */
dg_status dg_model_create(const dg_model_desc* desc, const dg_weights* w, dg_model** out);
void dg_model_destroy(dg_model* m);

/* Replay each step as a captured hipGraph (default on).  Applies to
 * dg_denoise_step and dg_generate_block on a non-default stream; the default
 * stream cannot be captured and always runs the kernels directly.  Graphs are
 * cached per distinct argument set (up to 8) and freed by dg_model_destroy. */
dg_status dg_set_graphs(dg_model* m, int32_t enable);

/* Bytes of the key/value cache for Bp prefixes of capacity P_max:
 * per layer K [Bp][Hkv][P_max][hd] then V^T [Bp][Hkv][P_max / 32][hd][32] (tile-major:
 * position p of dim d at ((p / 32) hd + d) 32 + p % 32, each 32-key tile one contiguous
 * block), bf16. */
size_t dg_kv_bytes(const dg_model* m, int32_t Bp, int32_t P_max);

/* Workspace bytes for passes over up to `rows` token rows attending up to
 * `keys` keys (rows = B*T and keys = P + T for a step; a prefill uses chunks
 * of at most `rows` tokens of a prefix of at most `keys` tokens). */
size_t dg_workspace_bytes(const dg_model* m, int32_t rows, int32_t keys);

/* Causal encoding of Bp prompts.  prefix: int32 [Bp][P] token ids (or, for
 * dg_prefill_hidden, fp32 [Bp][P][d] input hidden states).  Writes K (after
 * QK-norm and RoPE) and V of positions 0..P-1 of every layer into kv.  The
 * prefix is processed in chunks of the largest row count the workspace allows. */
dg_status dg_prefill_prefix(dg_model* m, const int32_t* prefix, int32_t Bp, int32_t P, int32_t P_max, void* kv,
                            void* ws, size_t ws_bytes, dg_stream_t stream);
dg_status dg_prefill_hidden(dg_model* m, const float* prefix_hidden, int32_t Bp, int32_t P, int32_t P_max,
                            void* kv, void* ws, size_t ws_bytes, dg_stream_t stream);

/* Block continuation (the finished block joins the causally encoded prompt,
 * article section 2 and section 5): encodes tokens int32 [Bp][n] at positions
 * P0 .. P0+n-1 of each prompt, attending causally to the K/V of positions
 * 0 .. P0-1 already in kv and to each other, and writes their K and V into kv.
 * dg_prefill_prefix is the case P0 = 0.  Any P0 >= 0 and n >= 1 with
 * P0 + n <= P_max (else DG_ERR_ARG before any device work); a denoising step
 * over the result needs P0 + n to be a multiple of 32. */
dg_status dg_prefill_append(dg_model* m, const int32_t* tokens, int32_t Bp, int32_t P0, int32_t n, int32_t P_max,
                            void* kv, void* ws, size_t ws_bytes, dg_stream_t stream);

/* dg_prefill_append that also records, for the positions dump_pos ..
 * dump_pos + dump_n - 1 of prompt 0 (inside [P0, P0 + n)), the input of every
 * layer and the final hidden state, hidden_dump fp32 [n_layers + 1][dump_n][d],
 * and the routing of every layer: expert_dump int32 [n_layers][dump_n][top_k],
 * gate_dump fp32 of the same shape, router_dump fp32 [n_layers][dump_n]
 * [n_experts] (any of them may be NULL).  For parity checks of the prompt
 * cache at the model's full depth.  The recorded positions are encoded as one
 * pass, so dump_n must not exceed the largest pass the workspace allows
 * (DG_ERR_WORKSPACE otherwise); the cache written is the same as
 * dg_prefill_append's. */
dg_status dg_prefill_dump(dg_model* m, const int32_t* tokens, int32_t Bp, int32_t P0, int32_t n, int32_t P_max,
                          void* kv, int32_t dump_pos, int32_t dump_n, float* hidden_dump, int32_t* expert_dump,
                          float* gate_dump, float* router_dump, void* ws, size_t ws_bytes, dg_stream_t stream);

/* One autoregressive decoding step (the model still generates token by token:
 * arXiv abstract page; article section 5 compares a denoising step with this
 * one) for B sequences with caches kv [B] of capacity P_max:
 *   - token int32 [B] (device): the token at position P of each sequence; it
 *     is encoded against the cached positions 0..P-1 and its K/V written at P;
 *   - then the final norm, the LM head and the next token
 *       next[b] = argmax_v fp32(l_v * inv_tau) + G_v   (ties -> lowest v),
 *     inv_tau = fp32(1 / tau) taken in double, G_v the Gumbel variate of word
 *     v & 3 of Philox4x32-10 block (v >> 2, P, 0, 2) keyed by row_seeds[b]
 *     (host [B]): a sample of softmax(l / tau);
 *   - argmax [B] (argmax of the logits), entropy [B] (nats, of softmax(l)) and
 *     logits_dump fp32 [B][V] are optional outputs (NULL to skip).
 * `next` may be the `token` buffer (the next call then reads it).  Sequences
 * run one after another, each one row through every layer.  On a non-default
 * stream (graphs enabled) the step is a captured hipGraph: P is written to
 * the workspace and read on the device, so calls that differ only in P (for
 * example decoding in place, token == next) replay one graph.  Needs
 * dg_workspace_bytes(m, 1, P + 1).  B in 1..16, P + 1 <= P_max, tau > 0,
 * vocab a multiple of 4; else a negative status before any device work. */
dg_status dg_ar_step(dg_model* m, void* kv, int32_t B, int32_t P, int32_t P_max, const int32_t* token, float tau,
                     const uint64_t* row_seeds, int32_t* next, int32_t* argmax, float* entropy, float* logits_dump,
                     void* ws, size_t ws_bytes, dg_stream_t stream);

/* Layer stack on canvas hidden states: hidden fp32 [B][T][d] in/out (input of
 * layer 0 in, output of the last layer out), bidirectional over the canvas and
 * attending all P prefix keys of prefix (Bp == 1 ? 0 : b).  Dumps as in
 * dg_canvas (may be NULL). */
dg_status dg_forward_hidden(dg_model* m, const void* kv, int32_t Bp, int32_t P, int32_t P_max, int32_t B,
                            int32_t T, float* hidden, float* hidden_dump, int32_t* expert_dump, float* gate_dump,
                            void* ws, size_t ws_bytes, dg_stream_t stream);

/* One denoising step at step index `step` (>= 0) for B canvases: embedding
 * + self-conditioning, all layers, final norm, LM head, entropy, Gumbel-max
 * sample, lock, re-randomisation, stop decision, soft-prediction embedding.
 * Sets steps[b] = step + 1 and stopped[b] for every row not already stopped. */
dg_status dg_denoise_step(dg_model* m, const void* kv, int32_t Bp, int32_t P, int32_t P_max, int32_t B, int32_t T,
                          dg_canvas* canvas, int32_t step, const dg_sampler* sp, void* ws, size_t ws_bytes,
                          dg_stream_t stream);

/* A whole block: resets stopped/steps/self_cond, then runs steps 0, 1, ...
 * until every row has stopped or max_steps is reached.  The step index lives
 * on the device (steps[b]); the host checks for an early stop every
 * `poll_every` steps (0 = never; the remaining launches then exit at once). */
dg_status dg_generate_block(dg_model* m, const void* kv, int32_t Bp, int32_t P, int32_t P_max, int32_t B,
                            int32_t T, dg_canvas* canvas, const dg_sampler* sp, int32_t poll_every, void* ws,
                            size_t ws_bytes, dg_stream_t stream);

/* The sampler alone on caller-given logits fp32 [B][T][V] (row pitch V):
 * entropy, Gumbel-max sample, lock, re-randomisation, stop, exactly as inside
 * dg_denoise_step.  Needs dg_sample_workspace_bytes(B, T, V) of workspace. */
size_t dg_sample_workspace_bytes(int32_t B, int32_t T, int32_t V);
dg_status dg_sample_logits(const float* logits, int32_t B, int32_t T, int32_t V, dg_canvas* canvas, int32_t step,
                           const dg_sampler* sp, void* ws, size_t ws_bytes, dg_stream_t stream);

/* The sampler of dg_sample_logits for callers that cannot allocate device
 * memory (code under stream capture, serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the per-slice partials in a
 * scratch area the library owns (a static device array of
 * dg_sample_noalloc_max_bytes() = 1 MiB on each GPU it runs on, kept until
 * the process ends).  Runs on the current device; `stream` must belong to it.
 * No allocation of any kind.  Every call on one GPU shares that GPU's area, so
 * calls that overlap on one GPU (different streams, or different host threads)
 * race: order them.  Nothing in the area needs clearing between calls (every
 * partial a call reads is written by that call).  Requests larger than the
 * area return DG_ERR_WORKSPACE before any device work (none of the accepted
 * shapes is: B <= 16, T <= 1024 needs at most 768 KB). */
size_t dg_sample_noalloc_max_bytes(void);
dg_status dg_sample_logits_noalloc(const float* logits, int32_t B, int32_t T, int32_t V, dg_canvas* canvas,
                                   int32_t step, const dg_sampler* sp, dg_stream_t stream);

/* Initial canvas: tokens[b][i] uniform over the vocabulary from Philox counter
 * (i, 0, 0xFFFFFFFF, 1) keyed by row_seeds[b]; also zeroes stopped, steps,
 * argmax and (if not NULL) self_cond. */
dg_status dg_init_canvas(const dg_model* m, dg_canvas* canvas, int32_t B, int32_t T, const uint64_t* row_seeds,
                         dg_stream_t stream);

/* C fp32 [M][N] (row pitch ldc) = A [M][K] (bf16, pitch lda) times W^T, W bf16
 * [N][K] (pitch ldw): the MFMA weight-streaming GEMM every projection of the
 * step uses, exposed on its own (M >= 192 runs on the 256 x 256 tile kernel,
 * 128 <= M < 192 on the 8-wave 64-row one, smaller M on the 4-wave one).  K a multiple of 64; lda and ldw multiples of
 * 8 (16-byte aligned rows), else DG_ERR_SHAPE before any device work. */
dg_status dg_gemm_bf16(const void* A, int64_t lda, const void* W, int64_t ldw, int32_t M, int32_t N, int32_t K,
                       float* C, int64_t ldc, dg_stream_t stream);

/* C fp32 [M][N] (row pitch ldc) = A [M][K] (bf16, pitch lda) times W [K][N]
 * (bf16, pitch ldw: the weight stored K-major, N values per row), the product
 * the soft-prediction embedding forms with the tied embedding E [vocab][d] as
 * stored (K = vocabulary, N = d).  256 x 256 tiles; the B operand is read
 * from LDS with gfx950 transposed loads.  K a multiple of 64; N, lda and ldw
 * multiples of 8; 256 lda and 64 ldw + N under 2^30 elements; else
 * DG_ERR_SHAPE before any device work. */
dg_status dg_gemm_bf16_kn(const void* A, int64_t lda, const void* W, int64_t ldw, int32_t M, int32_t N, int32_t K,
                          float* C, int64_t ldc, dg_stream_t stream);


/* Timing of kernel classes with HIP events recorded around their launches
 * (for measurement; adds event records to the stream while enabled).
 * dg_profile_enable(m, 1) clears the records and starts recording;
 * dg_profile_read waits for the recorded events and returns the summed
 * elapsed milliseconds and the number of launch groups of class `cls`.
 * Launches keep their streams while recording (the shared FFN and the
 * Gumbel pass run on the side stream), so classes on the two streams overlap
 * in time and their sums may exceed the step's wall time. */
enum {
  DG_PROF_DENSE = 0,          /* QKV and O projections, self-conditioning projection */
  DG_PROF_ATTN = 1,           /* attention partials + merge                          */
  DG_PROF_ROUTER = 2,         /* router logits, top-k, expert permutation            */
  DG_PROF_EXPERT_GATEUP = 3,  /* grouped expert gate/up GEMM with GELU-gating         */
  DG_PROF_EXPERT_DOWN = 4,    /* grouped expert down GEMM                            */
  DG_PROF_SHARED = 5,         /* shared FFN                                          */
  DG_PROF_LMHEAD = 6,         /* LM-head logits GEMM                                 */
  DG_PROF_SAMPLER = 7,        /* entropy / Gumbel / lock / stop                       */
  DG_PROF_SOFTEMB = 8,        /* soft-prediction embedding                           */
  DG_PROF_OTHER = 9,          /* norms, RoPE, combine                                */
  DG_PROF_NCLASS = 10
};
dg_status dg_profile_enable(dg_model* m, int32_t on);
dg_status dg_profile_read(dg_model* m, int32_t cls, double* total_ms, int32_t* count);

/* Host-side reference entry points of the library's own sampler arithmetic
 * (same source as the device code; no GPU needed): Philox4x32-10 block,
 * fp32 log, Gumbel variate of a 32-bit word, 1/tau of a step. */
void dg_host_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
float dg_host_ln(float x);
float dg_host_gumbel_of_word(uint32_t word);
float dg_host_inv_tau(float tau_start, float tau_end, int32_t max_steps, int32_t step);
/* Batched forms over n host values: out[i] = ln(x[i]); out[i] = Gumbel(word[i]). */
void dg_host_ln_batch(const float* x, float* out, int64_t n);
void dg_host_gumbel_batch(const uint32_t* words, float* out, int64_t n);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
