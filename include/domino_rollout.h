/*
 * domino_rollout.h — C ABI of the MI355X (gfx950) Domino draft-block rollout.
 *
 * What is computed (sources cited by page title and section):
 *   "Add correctness-first Domino support to DFlash V2" (sglang PR #31328),
 *   section "Design": for a draft block of 16 positions the rollout emits 15
 *   proposals per request.  Proposal 1 is the full-vocabulary argmax of the
 *   base LM-head logits; a bias-free GRU is seeded with
 *   [verified_token, proposal 1]; each later proposal is the argmax of
 *   base logits plus a per-step correction, taken over the full vocabulary
 *   (K = 0) or over one per-request, block-shared pool of the K best ids;
 *   every chosen token is fed back into the GRU before the next step.
 *   "[Spec] Add Domino projector support to DFlash speculative decoding (V2)"
 *   (sglang PR #28998), sections "Motivation" and "Implementation": the
 *   correction is SiLU(z + s)·fc2ᵀ + bias added to the lm_head logits.
 *   "feat: support tensor-parallel Domino rollout" (sglang PR #32018),
 *   section "Implementation": proposal 1 stays a full-vocabulary argmax; the
 *   lm_head is the target model's, shared rather than copied.
 *
 * Exact arithmetic of one run (all accumulation in fp32):
 *   base[t,b,v] = sum_i hidden[b,t,i] * lm_head[v,i]              t = 0..14
 *   p[b,1]      = argmax_v base[0,b,v]
 *   pool C_b    = all ids                      if K == 0 or K >= V
 *               = K ids with the largest max_t base[t,b,v], ties to the
 *                 lower id                     if 0 < K < V
 *   h = 0;  h = GRU(E[verified[b]], h);  h = GRU(E[p[b,1]], h)
 *   for k = 1..14:
 *     u = SiLU(fc1_w · h + step_s[b,k-1,:])
 *     y_c = base[k,b,c] + (fc2_w[c,:] · u + fc2_b[c])      for c in C_b
 *     p[b,k+1] = argmax_c y_c  (ties to the lower id; -0.0 == +0.0)
 *     if k < 14: h = GRU(E[p[b,k+1]], h)
 *   GRU(x, h): a = W_ih x, c = W_hh h, rows ordered (r, z, n), no biases;
 *     r = sigmoid(a_r + c_r), z = sigmoid(a_z + c_z),
 *     n = tanh(a_n + r * c_n), h' = (1 - z) * n + z * h.
 *
 * Threading / streams: a handle is not re-entrant (one run in flight per
 * handle).  Every run enqueues its kernels on the caller's stream and
 * returns without a host synchronisation.  domino_rollout_run never
 * allocates device memory, so a caller may capture it into its own graph.
 */
#ifndef DOMINO_ROLLOUT_H
#define DOMINO_ROLLOUT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DOMINO_OK = 0,
  DOMINO_ERR_INVALID_ARG = -1,     /* bad scalar or NULL pointer; nothing launched */
  DOMINO_ERR_INVALID_CONFIG = -2,  /* create(): inconsistent configuration        */
  DOMINO_ERR_UNSUPPORTED = -3,     /* device is not gfx950, or a shape the library
                                      does not handle (see domino_config_t)       */
  DOMINO_ERR_OUT_OF_MEMORY = -4,   /* workspace allocation failed in create()      */
  DOMINO_ERR_HIP = -5              /* a HIP runtime call failed                    */
} domino_status_t;

typedef enum { DOMINO_DTYPE_BF16 = 0, DOMINO_DTYPE_FP32 = 1 } domino_dtype_t;

/* Mirrors the Domino fields of the draft configuration ("[Spec] Add Domino
 * projector support ..." section "Implementation": gru_hidden_dim, emb_dim,
 * pure_draft_prefix_len; block size 16 per "Add correctness-first Domino
 * support ..." section "Supported and numerical scope").  Validated by
 * domino_rollout_create. */
typedef struct {
  int32_t vocab;        /* V  > 0                                              */
  int32_t hidden;       /* H  > 0, multiple of 64                              */
  int32_t emb_dim;      /* e  > 0, multiple of 32                              */
  int32_t gru_hidden;   /* g  > 0, multiple of 32                              */
  int32_t proj_dim;     /* r  > 0, multiple of 32                              */
  int32_t block_size;   /* must be 16: 15 proposals, 14 correction steps       */
  int32_t pure_draft_prefix_len; /* must be 1                                  */
  int32_t max_batch;    /* 1..64: workspace is sized for this many requests    */
  int32_t max_k;        /* >= 0: largest pool size run() accepts (0 = no pool) */
  int32_t dtype;        /* domino_dtype_t of weights and hiddens               */
} domino_config_t;

/* BORROWED device pointers (row-major, dtype of the config) that must stay
 * valid and unchanged for the life of the handle. */
typedef struct {
  const void* lm_head;   /* [V, H]  the target model's LM head                 */
  const void* embed;     /* [V, e]  token embedding feeding the GRU            */
  const void* gru_w_ih;  /* [3g, e] rows ordered (r, z, n), bias-free          */
  const void* gru_w_hh;  /* [3g, g] rows ordered (r, z, n), bias-free          */
  const void* fc1_w;     /* [r, g]  projector layer 1 (GRU half)               */
  const void* fc2_w;     /* [V, r]  projector layer 2                          */
  const void* fc2_b;     /* [V]     projector layer 2 bias                     */
  /* Optional (both or neither; NULL: the caller passes step_s to every run):
   * the backbone-hidden half of projector layer 1 and that layer's bias.
   * With them a run may pass step_s = NULL and the library forms
   * step_s[b, j, :] = fc1_x_w · base_hidden[b, j+1, :] + fc1_b itself
   * (projector input [backbone hidden | GRU state], "Add correctness-first
   * Domino support to DFlash V2", commit text). */
  const void* fc1_x_w;   /* [r, H]  projector layer 1 (backbone-hidden half)   */
  const void* fc1_b;     /* [r]     projector layer 1 bias                     */
} domino_weights_t;

typedef struct domino_rollout domino_rollout_t;

/* Validates the configuration, checks that the current HIP device is gfx950,
 * records the borrowed weights and allocates the workspace (base logits
 * [15, max_batch, V] fp32, pool buffers, GRU / projector state).  It also
 * forms, once, the GRU input projection of every vocabulary id,
 * G[v, :] = gru_w_ih · embed[v, :] ([V, 3g] fp32, 1.9 GB at V = 151936,
 * g = 1024), so that a GRU update reads one row of G instead of multiplying
 * gru_w_ih by an embedding row, and keeps repacked copies of [fc1_w; gru_w_hh]
 * (8.4 MB at g = r = 1024) and, when max_batch > 16, of fc2_w (311 MB at
 * V = 151936, r = 1024) in the order the matrix cores read them.  This is why
 * these weights must not change while the handle lives.  With bf16 weights,
 * max_batch >= 17 and H a multiple of 128, the workspace also holds the
 * block's hiddens in fragment order for the LM-head (8.4 MB at 64 requests,
 * H = 4096, rewritten by every run).  create()
 * synchronises the device.  On success
 * *out owns the handle; on failure *out is NULL and the status says why
 * (domino_rollout_last_error(NULL) holds the message). */
domino_status_t domino_rollout_create(const domino_config_t* cfg, const domino_weights_t* w,
                                      domino_rollout_t** out);

/* One rollout for `batch` requests, enqueued on `stream` (hipStream_t; NULL
 * = the default stream).  Device pointers, caller-owned:
 *   base_hidden     [batch, 15, H]  dtype of the config: the block's draft hiddens
 *   step_s          [batch, 14, r]  fp32: the backbone-hidden half of the
 *                                   projector input plus the fc1 bias, per step;
 *                                   NULL if the handle holds fc1_x_w / fc1_b
 *                                   (the library then computes it)
 *   verified_tokens [batch]         int32 in [0, V)
 *   out_tokens      [batch, 15]     int32: proposals 1..15
 *   out_top1_logit  [batch, 15]     fp32 or NULL: the winning logit of each
 *                                   proposal (column 0: base logit of p1)
 * K == 0 or K >= V selects the full vocabulary; 0 < K < V a pool of K ids
 * (K <= max_k).  Returns DOMINO_ERR_INVALID_ARG without launching anything
 * for batch outside [1, max_batch], K < 0, K > max_k with K < V, or a NULL
 * pointer.  A verified token outside [0, V) is not read; that request's
 * outputs become -1 (tokens) and NaN (logits). */
domino_status_t domino_rollout_run(domino_rollout_t* h, const void* base_hidden,
                                   const float* step_s, const int32_t* verified_tokens,
                                   int32_t batch, int32_t K, int32_t* out_tokens,
                                   float* out_top1_logit, void* stream);

/* Most graphs a handle keeps cached (domino_rollout_run_graph). */
#define DOMINO_GRAPH_CACHE_MAX 16

/* Same computation as domino_rollout_run, replayed from a HIP graph that the
 * handle captures on first use for each distinct (batch, K mode, proposals,
 * pointer set).  The first call for a new key captures and instantiates
 * (host work); later calls are a single hipGraphLaunch plus an event record.
 * The cache holds at most DOMINO_GRAPH_CACHE_MAX graphs: a new key beyond
 * that evicts the least recently used graph, after a host wait for that
 * graph's last replay to finish (normally long done), so a caller that
 * rotates more buffer sets than that pays a capture per rotation but never
 * grows the cache.  A replay leaves the workspace as its own run does
 * (domino_rollout_read_workspace reports the replayed run's shape).  Not for
 * use inside the caller's own stream capture: use domino_rollout_run there. */
domino_status_t domino_rollout_run_graph(domino_rollout_t* h, const void* base_hidden,
                                         const float* step_s, const int32_t* verified_tokens,
                                         int32_t batch, int32_t K, int32_t* out_tokens,
                                         float* out_top1_logit, void* stream);

/* Truncated rollout: only the first `proposals` (1..15) proposals, for a
 * target that verifies only the first positions of the block ("Qwen3.6-27B
 * checkpoint and full serving benchmark", Methods: b8 keeps the block-16
 * draft backbone and verifies the first 8 positions).  The base logits, the
 * first proposal and the pool are those of the whole block, and the run stops
 * after proposals - 1 correction steps, so the result equals the first
 * `proposals` columns of domino_rollout_run.  out_tokens and out_top1_logit
 * (or NULL) are [batch, proposals].  graph != 0 replays a HIP graph cached
 * per (batch, K mode, proposals, pointer set), as domino_rollout_run_graph
 * does.  Other arguments and errors as domino_rollout_run; proposals outside
 * [1, 15] is DOMINO_ERR_INVALID_ARG. */
domino_status_t domino_rollout_run_prefix(domino_rollout_t* h, const void* base_hidden,
                                          const float* step_s, const int32_t* verified_tokens,
                                          int32_t batch, int32_t K, int32_t proposals,
                                          int32_t* out_tokens, float* out_top1_logit,
                                          int32_t graph, void* stream);

/* Teacher-forced variant for testing: the GRU consumes forced_tokens[b, j]
 * (device, [batch, 15] int32, values in [0, V)) in place of proposal j+1,
 * while out_tokens / out_top1_logit still report each step's argmax.  This
 * lets every step's logits be compared even after two chains diverge. */
domino_status_t domino_rollout_run_forced(domino_rollout_t* h, const void* base_hidden,
                                          const float* step_s, const int32_t* verified_tokens,
                                          const int32_t* forced_tokens, int32_t batch, int32_t K,
                                          int32_t* out_tokens, float* out_top1_logit,
                                          void* stream);

/* Copies a workspace buffer of the last run into dst (device memory of at
 * least dst_bytes), stream-ordered on `stream`.  which: 0 = base logits fp32
 * [15, batch, V] (step-major), 1 = pool ids int32 [batch, K] sorted
 * ascending (pool runs only), 2 = step_s fp32 [batch, 14, r] as the library
 * computed it (runs with step_s = NULL only), 3 = int32 [ceil(batch / G)]
 * sizes of the pool unions of each group of G requests (pool runs that
 * streamed the unions: bf16 weights, batch <= 64; G = 32, or 24 or 16 when a
 * 32-request panel of u does not fit in LDS, e.g. 24 at r = 1280).  *bytes receives
 * the buffer's size for the last run; with dst == NULL nothing is copied.
 * INVALID_ARG if which is unknown or not available for the last run, no run
 * has happened, or dst_bytes is too small. */
domino_status_t domino_rollout_read_workspace(const domino_rollout_t* h, int32_t which, void* dst,
                                              size_t dst_bytes, size_t* bytes, void* stream);

/* Measurement support.  While enabled, every kernel that domino_rollout_run
 * and domino_rollout_run_forced launch carries a HIP event pair stamped by
 * that kernel's own dispatch (its start and end on the GPU, without launch
 * gaps); graph replays are not instrumented.  domino_rollout_kernel_times
 * waits for the pending events, adds the kernel durations to per-phase
 * totals and returns the total milliseconds and the number of phase
 * instances of one phase: 0 = LM-head GEMM, 1 = correction + argmax (full
 * vocabulary or pool), 2 = GRU gates (the prefix launch, and the separate
 * gate kernel of step paths 2 and 3), 3 = step product: projector layer 1 +
 * SiLU and W_hh of the new state (with the gates in path 1, and its split-sum
 * kernel where used), 4 = pool build (all its kernels), 5 = first-proposal
 * argmax, 6 = step offsets formed in the library.  which = -1 clears the
 * totals.  Timing changes no result. */
domino_status_t domino_rollout_set_timing(domino_rollout_t* h, int32_t enable);

/* How each correction step forms the GRU update and projector layer 1
 * (identical arithmetic, different kernels): 0 = automatic by batch (the
 * default), 1 = one launch whose workgroups each evaluate the GRU gates of
 * every request before multiplying their rows of [fc1; gru_w_hh] (bf16, at
 * most 8 requests), 2 = a gate kernel, then the same row product (bf16, at
 * most 16 requests), 3 = a gate kernel, then a matrix-core product.  Paths 1
 * and 2 fall back to 3 where they do not apply.  The paths sum in different
 * orders, so results may differ in the last bits of fp32.  Changing the path
 * waits for the device and drops the handle's cached graphs.  INVALID_ARG
 * for any other value. */
domino_status_t domino_rollout_set_step_path(domino_rollout_t* h, int32_t path);

/* How pool corrections (0 < K < V) read the fc2 rows when the batch has at
 * most 64 requests and the weights are bf16: 0 = automatic (the default:
 * group unions once the per-request gather would read 96 MB or more per step,
 * 48 MB at 16 requests or fewer), 1 = every request gathers its own K rows,
 * 2 = each group of 32 requests (24 or 16 for projectors too wide for a
 * 32-request panel in LDS) streams the union of its pools once (where the
 * projector width allows it: r a multiple of 256; otherwise the gather).  Both score the same candidates; their dot products are summed in
 * different orders, so top-1 values may differ in the last bits.  Changing
 * the strategy waits for the device and drops the handle's cached graphs.
 * INVALID_ARG for any other value.  ("feat: support tensor-parallel Domino
 * rollout", "Rollout performance": the candidate pool's gain shrinks at
 * batch 64, where the pools of a batch cover much of the vocabulary.) */
domino_status_t domino_rollout_set_pool_strategy(domino_rollout_t* h, int32_t strategy);
domino_status_t domino_rollout_kernel_times(domino_rollout_t* h, int32_t which, double* total_ms,
                                            int64_t* launches);

/* Size of the library's static scratch array on each device (bytes). */
#define DOMINO_STATIC_SCRATCH_BYTES (6u << 20)

/* For callers that cannot allocate device memory at run time (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same rollout as domino_rollout_run (same kernels, bit-identical
 * results), whose per-run scratch -- argmax words, bad-request flags, radix
 * histograms / state, GRU state and W_hh h, u and its bf16
 * planes, the fragment-ordered state and split partials -- lives in one
 * static device array of DOMINO_STATIC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends, instead of the
 * handle's workspace.  The call allocates nothing; the handle (created
 * beforehand, which does allocate) still holds the base logits, pool and
 * the tables formed at create.  Each call first clears the part of the array
 * it uses with a fill kernel, then enqueues the rollout on `stream`.  Every
 * call on one device shares that device's array: calls whose work overlaps
 * on one device (other streams, other handles, other threads) race and give
 * undefined results; serialise them.  The scratch needed grows with the
 * batch (about 85 KB per request plus 1 MB at g = r = 1024, so up to ~58
 * requests there); a batch whose scratch exceeds the array is
 * DOMINO_ERR_INVALID_ARG and nothing is launched.  Other arguments and
 * errors as domino_rollout_run (DOMINO_ERR_UNSUPPORTED if the array's
 * device address could not be looked up at create). */
domino_status_t domino_rollout_run_static(domino_rollout_t* h, const void* base_hidden,
                                          const float* step_s, const int32_t* verified_tokens,
                                          int32_t batch, int32_t K, int32_t* out_tokens,
                                          float* out_top1_logit, void* stream);

/* Number of graphs the handle has cached (0..DOMINO_GRAPH_CACHE_MAX) in
 * *count.  INVALID_ARG for a NULL handle or count. */
domino_status_t domino_rollout_cached_graphs(const domino_rollout_t* h, int32_t* count);

/* Frees the workspace and cached graphs (not the borrowed weights). NULL is a no-op. */
void domino_rollout_destroy(domino_rollout_t* h);

/* Message of the handle's last error, or of the last failed create() when
 * h is NULL.  Never NULL; "" when there was no error. */
const char* domino_rollout_last_error(const domino_rollout_t* h);

#ifdef __cplusplus
}
#endif
#endif /* DOMINO_ROLLOUT_H */
