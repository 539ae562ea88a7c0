// Host-side launchers of the rollout kernels (internal interface between the
// orchestration in rollout.hip and the kernels in kernels.hip / lmhead.hip).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

// Kernel timing.  While a phase of a run is being timed on the calling
// thread, timing_events hands out an event pair that the launch attaches to
// the kernel's own dispatch (start and end stamps of that kernel alone);
// otherwise it returns false and the launch is a plain one.
bool timing_events(hipEvent_t* start, hipEvent_t* stop);
#define DLAUNCH(kernel, grid, block, shmem, stream, ...)                                          \
  do {                                                                                           \
    hipEvent_t dl_start_ = nullptr, dl_stop_ = nullptr;                                          \
    if (timing_events(&dl_start_, &dl_stop_))                                                    \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, dl_start_, dl_stop_, 0,          \
                            __VA_ARGS__);                                                        \
    else                                                                                         \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                       \
  } while (0)

struct DeviceWeights {
  const void* lm_head;
  const void* embed;
  const void* w_ih;
  const void* w_hh;
  const void* fc1;
  const void* fc2;
  const void* fc2_b;
  const void* fc1_x;  // optional backbone-hidden half of projector layer 1 [r, H]
  const void* fc1_b;  // optional projector layer 1 bias [r]
};

struct Shape {
  int V, H, e, g, r;
  bool bf16;
};

// workspace buffers of one handle
struct Workspace {
  float* base;         // [15, Bmax, V] step-major base logits
  uint32_t* keys;      // [Bmax, V] orderable pool scores
  uint32_t* hist;      // [Bmax, 3, 2048] radix histograms
  uint32_t* state;     // [Bmax, 4, 2] radix state (prefix, remaining count) after 0..2 selections
  int32_t* pool_ids;   // [Bmax, Kmax]
  uint2* cand;         // [Bmax, V] pool candidates (key, id), compacted per id chunk
  uint32_t* cand_n;    // [Bmax, nchunks] candidates per chunk of kPoolChunk ids
  float* pool_base;    // [14, Bmax, Kmax]
  float* h[2];         // [Bmax, g] ping-pong GRU state
  float* c[2];         // [Bmax, 3g] W_hh h of the matching state
  uint16_t* Wp;        // stacked [fc1; W_hh] in fragment order (bf16 models)
  uint16_t* hp;        // new state in fragment order, hi/lo bf16 (bf16 models)
  uint16_t* xp;        // the block's hiddens in fragment order for the LM-head above 24 requests
  uint16_t* fc2p;      // fc2 in tile order for the full-vocabulary stream (bf16, r % 128 == 0,
                       // max_batch >= kPackedStreamMinBatch)
  float* G;            // [V, 3g] GRU input projection of every id (built at create)
  float* u;            // [Bmax, r]
  uint16_t* u_hi;      // [Bmax, r]
  uint16_t* u_lo;      // [Bmax, r]
  uint64_t* slots;     // [15, Bmax] argmax words, kSlotSpan u64 each (common.h)
  int32_t* bad;        // [Bmax]
  float* partial;      // split partial tiles of the step product
  float* s_tmp;        // k-split partials of the step-offset product
  float* s;            // [Bmax, 14, r] per-step projector offsets formed in the library
  // pool rows streamed once per group of ugroup requests (bf16, large batches)
  uint32_t* umask;     // [ugmax, V] member bits of each id per group; zero between runs
  uint32_t* ucounts;   // [ugmax, nchunks, 2] (union rows, members) per id chunk
  uint4* urec;         // [ugmax, Umax] union rows in id order: {id, b2 as float bits,
                       // first member slot, member bits}
  int32_t* uidx;       // [ugmax, V] union row of an id (valid for the group's members)
  int32_t* un;         // [ugmax] union sizes
  float* mb;           // [14, ugmax, mstride] base logits of the members, union order
  int umax;            // Umax: rows per group list, min(V, ugroup * Kmax)
  int mstride;         // member slots per group, ugroup * Kmax
  int ugroup;          // requests per union group (at most kUnionGroup; 0: no unions)
  int ugmax;           // groups at max_batch
  int pool_strategy;   // 0 automatic, 1 per-request gather, 2 group unions where supported
};

// The full-vocabulary correction reads fc2 in tile order from this batch on.
// Measured at the 8B shapes (us per launch, tile order / row-major): B = 1
// 51.5 / 49.2, 8 53.6 / 51.5, 16 55.7 / 55.1, 24 61.7 / 62.8, 32 64.5 / 65.5,
// 48 71.2 / 86.6, 64 69.4 / 89.2.  Up to 16 requests every fc2 line crosses
// from L2 to the CUs once and row-major streams slightly faster; with two
// 32-request groups it crosses twice, and the fragment-shaped loads of the
// row-major layout limit that traffic.
constexpr int kPackedStreamMinBatch = 17;

// most requests per union group (one 32-bit member mask per union row); a
// projector too wide for a 32-request panel takes 24 or 16
constexpr int kUnionGroup = 32;

constexpr int kPoolChunk = 1024;
// pool selection passes take 4 x or 2 x kPoolChunk ids per workgroup from
// these batch sizes on
constexpr int kPoolChunk4MinBatch = 32;
constexpr int kPoolChunk2MinBatch = 16;

// streaming row kernel (stream.hip)
struct StreamArgs {
  const uint16_t* W;       // [N, K] bf16 weight rows, streamed once
  int N, K;
  const uint16_t* act_hi;  // activation rows, bf16
  const uint16_t* act_lo;  // low halves (correction) or nullptr
  int ncols;               // activation columns (<= 128)
  int col_B;               // > 0: column m reads row (m % col_B) * DOMINO_T + m / col_B
  int KS;                  // k slice staged in LDS (set by the launcher)
  float* out;              // store epilogue: [ncols, N]
  const uint16_t* b2;      // argmax epilogue: bias [N], base row [ncols, N], words [ncols]
  const float* base_k;
  uint64_t* slot_k;
  int reverse;             // walk k from the end (alternated between steps)
  int groups;              // column groups (set by the launcher)
  int gcols;               // columns per group (set by the launcher)
  // union epilogue: group g streams the rows of urec[g * ustride ..] (un[g]
  // of them) and folds only member pairs, with base values from mb_k
  const uint4* urec;
  const int32_t* un;
  const float* mb_k;       // [groups, mstride] for this step
  int ustride, mstride;
  int umaxu;               // units per wave staged in LDS (set by the launcher)
  // W repacked in tile order (launch_pack_tiles), or nullptr; the persistent
  // full-vocabulary argmax stream reads it instead of W
  const uint16_t* Wpk;
};
bool rowstream_supported(int K, int ncols);
// W [N, K] (K a multiple of 128) in tile order, N rounded up to 16 rows
size_t packed_tiles_elems(int N, int K);
void launch_pack_tiles(const uint16_t* W, int N, int K, uint16_t* out, hipStream_t st);
void rowstream_prepare();
void launch_rowstream_store(StreamArgs a, hipStream_t st);
void launch_rowstream_argmax(StreamArgs a, hipStream_t st);
// whether the union stream runs for K-wide rows, ncols requests and row
// lists of at most ubound rows (its 32-request panel and staged records fit)
bool rowstream_union_supported(int K, int ncols, int ubound, int group);
// largest union group (32, 24 or 16 requests) whose stream fits K-wide rows,
// up to max_batch requests and lists of min(V, group * max_k) rows; 0: none
int rowstream_union_group(int K, int V, int max_batch, int max_k);
void launch_rowstream_union(StreamArgs a, int ubound, int group, hipStream_t st);

// GRU update and projector layer 1 of one correction step (gru_step.hip).
// Stacked rows [fc1 (r rows); W_hh (3g rows)] are multiplied by the new state
// h: rows < r give u = SiLU(z + s) (and its bf16 hi/lo planes), the others
// c = W_hh h for the next step's gates.  The gates read a = W_ih E[token] from
// the table G built at create().
struct StepArgs {
  const void* F1;          // [r, g] projector layer 1 (GRU half), weight dtype
  const void* W_hh;        // [3g, g]
  const float* G;          // [V, 3g] W_ih E[v] for every id v
  const float* h_prev;     // [B, g] state before the update; nullptr: zero state
  const float* c_prev;     // [B, 3g] W_hh h_prev (ignored when h_prev is nullptr)
  float* h_new;            // [B, g] state after the update
  float* c_new;            // [B, 3g] W_hh h_new (written by the W_hh rows)
  const int32_t* tok_i32;  // token of request b at tok_i32[b * tok_stride] ...
  int tok_stride;
  const uint64_t* tok_key; // ... or the argmax word of request b
  int32_t* bad;            // [B]: set to 1 for a token outside [0, V)
  const float* s;          // [B, 14, r] projector offsets
  int step;                // s row (k - 1)
  float* u;                // [B, r]
  uint16_t* u_hi;          // [B, r] (bf16 models)
  uint16_t* u_lo;
  int row0, nrows;         // stacked rows [row0, row0 + nrows); multiples of 16
  float* partial;          // split partial tiles of the matrix-core path
  // bf16 matrix-core path: operands in fragment order (see gru_step.hip)
  const uint16_t* Wp;      // [(r + 3g) / 16][g / 32][64 lanes][8] stacked weights
  uint16_t* hp;            // [ceil(B / 16)][g / 32][hi, lo][64 lanes][8] new state, written
                           // by the gate kernel when not nullptr
  int B, V, g, r;
};
// arrangements of a step (see gru_step.hip)
constexpr int kStepAuto = 0;
constexpr int kStepFused = 1;  // gates evaluated inside the row kernel: one launch
constexpr int kStepRows = 2;   // gate kernel + row kernel
constexpr int kStepMfma = 3;   // gate kernel + matrix-core kernel
constexpr int kStepRowsMaxBatch = 16;      // the row kernels take at most this many requests
constexpr int kStepFusedMaxBatch = 8;      // ... and with the gates inside, this many
// Automatic choice, from a sweep at the 8B shapes (per-launch us, fused | gate + rows | gate +
// matrix cores): B = 1: 5.1 | 4.0 + 4.1 | 4.0 + 4.7; B = 2: 7.0 | 4.3 + 4.5 | 4.2 + 4.7;
// B = 4: 10.7 | 4.3 + 6.1 | 4.2 + 5.3; B = 8: 18.6 | 4.2 + 9.8 | 4.0 + 5.5.  The fused kernel
// repeats every request's gate arithmetic in each workgroup, so it wins only while that is
// cheaper than a launch; the row product never wins and is kept for forced use.
constexpr int kStepFusedAutoMaxBatch = 2;  // fused up to this batch, then matrix cores
constexpr int kStepRowsAutoMaxBatch = 0;
constexpr int kStepMaxSplit = 4;           // workgroups per 16-row tile along g, at most
// which arrangement runs for B requests (forced: one of the constants above;
// a forced row path falls back to the matrix cores where rows are unsupported)
int step_path(const Shape& s, int B, int forced);
// floats of split partials the matrix-core path may write
size_t step_partial_floats(int g, int r);
void step_prepare();
void launch_gru_gates(const StepArgs& a, hipStream_t st);
// [fc1; W_hh] (bf16) in fragment order for the matrix-core step product
size_t step_packed_weight_elems(int g, int r);
void launch_pack_step_weights(const Shape& s, const DeviceWeights& w, uint16_t* Wp, hipStream_t st);
void launch_step_product(const Shape& s, const StepArgs& a, int path, hipStream_t st);
// G[v, :] = W_ih E[v], [V, 3g] fp32 (kernels.hip)
void launch_gru_table(const Shape& s, const DeviceWeights& w, float* G, hipStream_t st);

// LM-head GEMM with fused pool-score keys and first-proposal argmax (lmhead_fused.hip)
struct FusedArgs {
  const uint16_t* W;   // lm_head [V, H]
  const uint16_t* X;   // hidden [B, 15, H]
  float* base;         // [15, B, V]
  uint32_t* keys;      // [B, V] orderable max over the block, or nullptr
  uint64_t* slots;     // argmax words of position 0 [B]
  int V, H, B;
  uint16_t* XP;        // workspace for the hiddens in fragment order (lmhead_xfrag_elems), or nullptr
};
// A single request streams lm_head once through the row kernel (8B, per
// block: 1.117 against 1.152 ms fused); from two requests on, the fused
// GEMM with the pool-key and first-proposal epilogue (B = 2: even at K0,
// 0.622 against 0.632 ms at K = 2048; B = 3: 1.223 against 1.232 ms).
constexpr int kFusedMinBatch = 2;
void lmhead_fused_prepare();
bool lmhead_fused_supported(int H);
void launch_lmhead_fused(const FusedArgs& a, hipStream_t st);
// From 17 to 32 requests and at 56-64 (H a multiple of 128) the LM-head reads
// the hiddens from a fragment-ordered copy of lmhead_xfrag_elems(B, H) bf16
// elements; possible: for some B <= max_batch.
bool lmhead_xfrag_used(int B, int H);
bool lmhead_xfrag_possible(int max_batch, int H);
size_t lmhead_xfrag_elems(int B, int H);

void launch_lmhead(const Shape& s, const void* W, const void* X, float* out, int B, hipStream_t st);
// One-request LM-head with whole-line lm_head loads (lmhead_one.hip): base
// logits [15, 1, V], the pool score keys (when keys is not nullptr), their
// first radix histogram added into hist0 [2048] (when not nullptr; zero
// before) and the first-proposal argmax word *slot0; bf16, H a multiple of
// 1024 up to 5120 and V small enough for one CU's share of tiles to stay in
// LDS.
bool lmhead_one_supported(int V, int H);
int cu_count();
void lmhead_one_prepare();
void launch_lmhead_one(const uint16_t* W, const uint16_t* X, float* out, uint32_t* keys,
                       uint32_t* hist0, uint64_t* slot0, int V, int H, hipStream_t st);
void launch_row0_argmax(const Shape& s, const float* base, int B, uint64_t* slots, hipStream_t st);
// Whether a pool correction of B requests streams each request group's
// union of pool rows once (instead of gathering every request's rows).
bool pool_union(const Shape& s, const Workspace& ws, int B, int K);
// keys_ready: the per-id scores were already written by the fused LM-head;
// hist_ready: and their first radix histogram (the one-request LM-head);
// with pool_union(), also the per-group unions and member base values
void launch_pool_build(const Shape& s, const Workspace& ws, const void* fc2_b, int B, int K,
                       bool keys_ready, bool hist_ready, hipStream_t st);
void launch_correct_full(const Shape& s, const DeviceWeights& w, const Workspace& ws, int k, int B,
                         hipStream_t st);
void launch_correct_pool(const Shape& s, const DeviceWeights& w, const Workspace& ws, int k, int B,
                         int K, hipStream_t st);
// step_s[b, j, :] = fc1_x · X[b, j+1, :] + fc1_b into ws.s; the k-split
// partials (when batches are small) go to ws.s_tmp, which holds
// step_offsets_partial_floats(max_batch, H, r) floats
size_t step_offsets_partial_floats(int Bmax, int H, int r);
void launch_step_offsets(const Shape& s, const DeviceWeights& w, const void* X, const Workspace& ws,
                         int B, hipStream_t st);
// tokens and top-1 logits of proposals 1..P, [B, P]; then clears the argmax
// words, bad flags and (pool runs) radix histograms for the next run
void launch_writeout(const Workspace& ws, int B, int P, bool pool, int32_t* out_tokens,
                     float* out_top1, hipStream_t st);
