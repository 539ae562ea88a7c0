// C ABI of the Domino draft-block rollout: validation, workspace, launch
// order, graph cache.  The order of work follows "Add correctness-first
// Domino support to DFlash V2" (sglang PR #31328), "Design":
//   base logits (once per block) -> p1 = full-vocabulary argmax
//   -> [pool of K ids]  -> GRU(verified) -> GRU(p1)
//   -> 14 x { u = SiLU(fc1 h + s) ; corrected argmax ; GRU(new token) }
// with no GRU update after the last step (2 prefix + 13 feedback updates).
// On the GPU each GRU update is evaluated in the launch that needs its
// result (gru_step.hip): the prefix launch forms GRU(verified) and W_hh of
// it, and correction step k's first launch forms the update by p_k, then
// projector layer 1 and W_hh of the new state.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/domino_rollout.h"
#include "common.h"
#include "launch.h"

namespace {

std::mutex g_err_mu;
std::string g_err;  // last create() failure

void set_global_err(const std::string& s) {
  std::lock_guard<std::mutex> lk(g_err_mu);
  g_err = s;
}

struct GraphKey {
  int B, K, forced, P;
  const void* p[6];
  bool operator==(const GraphKey& o) const {
    if (B != o.B || K != o.K || forced != o.forced || P != o.P) return false;
    for (int i = 0; i < 6; ++i)
      if (p[i] != o.p[i]) return false;
    return true;
  }
};

// A cached graph, with the run shape its capture recorded (what
// read_workspace reports after a replay of it) and an event recorded after
// each of its launches, so that an evicted graph is destroyed only once its
// last replay has finished.
struct GraphEntry {
  GraphKey key;
  hipGraphExec_t exec;
  hipEvent_t done;
  uint64_t used;  // cache clock of the last use (least recently used is evicted)
  int last_B, last_K;
  bool last_union, last_s_internal;
};

// Scratch of the allocation-free runs (domino_rollout_run_static): the
// per-run buffers of a rollout (argmax words, bad-request flags, radix
// histograms / state, GRU state and W_hh h ping-pong, u and its
// bf16 planes, the fragment-ordered state, split partials) carved from one
// file-scope device array instead of the handle's workspace.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in):
// create() looks up its device address once per device with
// hipGetSymbolAddress, and the runs use that address.
constexpr size_t kStaticScratchBytes = (size_t)DOMINO_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, nullptr until looked up

// once per device, with that device current
bool static_scratch_init(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev]) return true;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return false;
  g_scratch_ptr[dev] = p;
  return true;
}

void* static_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[dev];
}

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kPhases = 7;
enum Phase { kLmHead = 0, kCorrect = 1, kGru = 2, kStep = 3, kPool = 4, kArgmax0 = 5, kOffsets = 6 };

}  // namespace

struct domino_rollout {
  domino_config_t cfg;
  DeviceWeights w;
  Shape shape;
  int device;
  Workspace ws;
  std::vector<void*> allocations;
  std::vector<GraphEntry> graphs;  // at most DOMINO_GRAPH_CACHE_MAX
  uint64_t graph_clock = 0;
  hipStream_t capture_stream = nullptr;
  int last_B = 0, last_K = 0;  // shape of the last enqueued run
  bool last_s_internal = false;  // the last run formed step_s itself
  bool last_union = false;       // the last run streamed the pool rows as group unions
  int step_path = kStepAuto;     // arrangement of the GRU / projector step (set_step_path)
  // measurement: kernel event pairs of the timed phases (see PhaseTimer)
  bool timing = false;
  bool capturing = false;
  struct Pending {
    int phase;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> free_events;
  double phase_ms[kPhases] = {};
  int64_t phase_n[kPhases] = {};

  hipEvent_t take_event() {
    if (!free_events.empty()) {
      hipEvent_t e = free_events.back();
      free_events.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  std::string err;

  domino_status_t fail(domino_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    err = buf;
    return st;
  }
};

static domino_status_t validate_config(const domino_config_t* c, std::string& why) {
  char buf[256];
  auto bad = [&](const char* msg) {
    why = msg;
    return DOMINO_ERR_INVALID_CONFIG;
  };
  if (c->vocab <= 0 || c->hidden <= 0 || c->emb_dim <= 0 || c->gru_hidden <= 0 || c->proj_dim <= 0)
    return bad("vocab, hidden, emb_dim, gru_hidden and proj_dim must be positive");
  if (c->block_size != 16) {
    snprintf(buf, sizeof buf, "block_size must be 16 (got %d)", c->block_size);
    return bad(buf);
  }
  if (c->pure_draft_prefix_len != 1) {
    snprintf(buf, sizeof buf, "pure_draft_prefix_len must be 1 (got %d)", c->pure_draft_prefix_len);
    return bad(buf);
  }
  if (c->max_batch < 1 || c->max_batch > 64) return bad("max_batch must be in [1, 64]");
  if (c->max_k < 0) return bad("max_k must be >= 0");
  if (c->dtype != DOMINO_DTYPE_BF16 && c->dtype != DOMINO_DTYPE_FP32)
    return bad("dtype must be DOMINO_DTYPE_BF16 or DOMINO_DTYPE_FP32");
  if (c->hidden % 64 || c->emb_dim % 32 || c->gru_hidden % 32 || c->proj_dim % 32) {
    why = "hidden must be a multiple of 64 and emb_dim, gru_hidden, proj_dim multiples of 32";
    return DOMINO_ERR_UNSUPPORTED;
  }
  if ((long long)DOMINO_T * c->max_batch * (long long)c->vocab > (1LL << 31) - 1 ||
      (long long)c->vocab * c->hidden > (1LL << 40)) {
    why = "shape too large";
    return DOMINO_ERR_UNSUPPORTED;
  }
  return DOMINO_OK;
}

extern "C" domino_status_t domino_rollout_create(const domino_config_t* cfg,
                                                 const domino_weights_t* w,
                                                 domino_rollout_t** out) {
  if (!out) {
    set_global_err("create: out is NULL");
    return DOMINO_ERR_INVALID_ARG;
  }
  *out = nullptr;
  if (!cfg || !w) {
    set_global_err("create: cfg or weights is NULL");
    return DOMINO_ERR_INVALID_ARG;
  }
  std::string why;
  domino_status_t st = validate_config(cfg, why);
  if (st != DOMINO_OK) {
    set_global_err("create: " + why);
    return st;
  }
  const void* wp[7] = {w->lm_head, w->embed, w->gru_w_ih, w->gru_w_hh, w->fc1_w, w->fc2_w, w->fc2_b};
  for (int i = 0; i < 7; ++i) {
    if (!wp[i]) {
      set_global_err("create: a weight pointer is NULL");
      return DOMINO_ERR_INVALID_ARG;
    }
    if (i < 6 && ((uintptr_t)wp[i] & 15)) {
      set_global_err("create: weight matrices must be 16-byte aligned");
      return DOMINO_ERR_INVALID_ARG;
    }
  }
  if ((w->fc1_x_w == nullptr) != (w->fc1_b == nullptr)) {
    set_global_err("create: fc1_x_w and fc1_b must be given together");
    return DOMINO_ERR_INVALID_ARG;
  }
  if (w->fc1_x_w && ((uintptr_t)w->fc1_x_w & 15)) {
    set_global_err("create: weight matrices must be 16-byte aligned");
    return DOMINO_ERR_INVALID_ARG;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_global_err("create: no HIP device");
    return DOMINO_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    set_global_err("create: hipGetDeviceProperties failed");
    return DOMINO_ERR_HIP;
  }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    set_global_err(std::string("create: device is ") + prop.gcnArchName + ", the library runs on gfx950 only");
    return DOMINO_ERR_UNSUPPORTED;
  }

  if (!static_scratch_init(dev)) {
    set_global_err("create: looking up the static scratch array failed");
    return DOMINO_ERR_HIP;
  }

  domino_rollout* h = new domino_rollout();
  h->cfg = *cfg;
  h->w = DeviceWeights{w->lm_head, w->embed, w->gru_w_ih, w->gru_w_hh, w->fc1_w,
                       w->fc2_w,   w->fc2_b, w->fc1_x_w,  w->fc1_b};
  h->shape = Shape{cfg->vocab, cfg->hidden, cfg->emb_dim, cfg->gru_hidden, cfg->proj_dim,
                   cfg->dtype == DOMINO_DTYPE_BF16};
  h->device = dev;

  const size_t V = cfg->vocab, Bm = cfg->max_batch, Km = cfg->max_k > 0 ? cfg->max_k : 1;
  const size_t g = cfg->gru_hidden, r = cfg->proj_dim;
  const size_t nch = (V + kPoolChunk - 1) / kPoolChunk;
  auto alloc = [&](size_t bytes) -> void* {
    void* p = nullptr;
    if (hipMalloc(&p, bytes < 256 ? 256 : bytes) != hipSuccess) return nullptr;
    h->allocations.push_back(p);
    return p;
  };
  Workspace& ws = h->ws;
  ws.base = (float*)alloc(DOMINO_T * Bm * V * 4);
  ws.keys = (uint32_t*)alloc(Bm * V * 4);
  ws.hist = (uint32_t*)alloc(Bm * 3 * 2048 * 4);
  ws.state = (uint32_t*)alloc(Bm * 8 * 4);
  ws.pool_ids = (int32_t*)alloc(Bm * Km * 4);
  if (cfg->max_k > 0) {
    ws.cand = (uint2*)alloc(Bm * V * 8);
    ws.cand_n = (uint32_t*)alloc(Bm * nch * 4);
  }
  ws.pool_base = (float*)alloc(DOMINO_S * Bm * Km * 4);
  ws.h[0] = (float*)alloc(Bm * g * 4);
  ws.h[1] = (float*)alloc(Bm * g * 4);
  ws.c[0] = (float*)alloc(Bm * 3 * g * 4);
  ws.c[1] = (float*)alloc(Bm * 3 * g * 4);
  ws.G = (float*)alloc(V * 3 * g * 4);
  const bool pack_fc2 =
      h->shape.bf16 && rowstream_supported((int)r, 1) && cfg->max_batch >= kPackedStreamMinBatch;
  if (h->shape.bf16) {
    ws.Wp = (uint16_t*)alloc(step_packed_weight_elems((int)g, (int)r) * 2);
    ws.hp = (uint16_t*)alloc((Bm + 15) / 16 * 16 * g * 4);
    if (pack_fc2) ws.fc2p = (uint16_t*)alloc(packed_tiles_elems((int)V, (int)r) * 2);
    const bool xfrag = lmhead_xfrag_possible((int)Bm, cfg->hidden);
    if (xfrag) ws.xp = (uint16_t*)alloc(lmhead_xfrag_elems((int)Bm, cfg->hidden) * 2);
    if (!ws.Wp || !ws.hp || (pack_fc2 && !ws.fc2p) || (xfrag && !ws.xp)) {
      set_global_err("create: workspace allocation failed");
      domino_rollout_destroy(h);
      return DOMINO_ERR_OUT_OF_MEMORY;
    }
  }
  ws.u = (float*)alloc(Bm * r * 4);
  ws.u_hi = (uint16_t*)alloc(Bm * r * 2);
  ws.u_lo = (uint16_t*)alloc(Bm * r * 2);
  ws.slots = (uint64_t*)alloc(DOMINO_T * Bm * kSlotSpan * 8);
  ws.bad = (int32_t*)alloc(Bm * 4);
  ws.partial = (float*)alloc(step_partial_floats((int)g, (int)r) * sizeof(float));
  if (h->w.fc1_x) {  // in-library step offsets
    ws.s_tmp = (float*)alloc(std::max<size_t>(step_offsets_partial_floats((int)Bm, cfg->hidden, (int)r), 64) *
                             sizeof(float));
    ws.s = (float*)alloc((size_t)DOMINO_S * Bm * r * sizeof(float));
  }
  // pool unions (pool_union()): groups of up to 32 requests, fewer when the
  // projector is too wide for a 32-request panel
  ws.ugroup = h->shape.bf16 ? rowstream_union_group((int)r, (int)V, (int)Bm, (int)Km) : 0;
  const bool unions = ws.ugroup > 0;
  if (unions) {
    const size_t G = (Bm + ws.ugroup - 1) / ws.ugroup;
    ws.ugmax = (int)G;
    ws.umax = (int)std::min<size_t>(V, (size_t)ws.ugroup * Km);
    ws.mstride = ws.ugroup * (int)Km;
    ws.umask = (uint32_t*)alloc(G * V * 4);
    ws.ucounts = (uint32_t*)alloc(G * nch * 2 * 4);
    ws.urec = (uint4*)alloc(G * (size_t)ws.umax * sizeof(uint4));
    ws.uidx = (int32_t*)alloc(G * V * 4);
    ws.un = (int32_t*)alloc(G * 4);
    ws.mb = (float*)alloc((size_t)DOMINO_S * G * ws.mstride * 4);
    if (!ws.umask || !ws.ucounts || !ws.urec || !ws.uidx || !ws.un || !ws.mb) {
      set_global_err("create: workspace allocation failed");
      domino_rollout_destroy(h);
      return DOMINO_ERR_OUT_OF_MEMORY;
    }
  }
  if (cfg->max_k > 0 && (!ws.cand || !ws.cand_n)) {
    set_global_err("create: workspace allocation failed");
    domino_rollout_destroy(h);
    return DOMINO_ERR_OUT_OF_MEMORY;
  }
  for (void* p : {(void*)ws.base, (void*)ws.keys, (void*)ws.hist, (void*)ws.state,
                  (void*)ws.pool_ids, (void*)ws.pool_base, (void*)ws.h[0], (void*)ws.h[1],
                  (void*)ws.c[0], (void*)ws.c[1], (void*)ws.G,
                  (void*)ws.u, (void*)ws.u_hi, (void*)ws.u_lo, (void*)ws.slots, (void*)ws.bad,
                  (void*)ws.partial, h->w.fc1_x ? (void*)ws.s : (void*)ws.partial,
                  h->w.fc1_x ? (void*)ws.s_tmp : (void*)ws.partial}) {
    if (!p) {
      set_global_err("create: workspace allocation failed");
      domino_rollout_destroy(h);
      return DOMINO_ERR_OUT_OF_MEMORY;
    }
  }
  // every buffer starts defined; the pool ids in particular are always valid rows
  for (size_t i = 0; i < h->allocations.size(); ++i) {
    if (hipMemset(h->allocations[i], 0, 256) != hipSuccess) break;
  }
  if ((unions && hipMemset(ws.umask, 0, (size_t)ws.ugmax * V * 4) != hipSuccess) ||
      (ws.hp && hipMemset(ws.hp, 0, (Bm + 15) / 16 * 16 * g * 4) != hipSuccess) ||
      hipMemset(ws.pool_ids, 0, Bm * Km * 4) != hipSuccess ||
      // cleared by every run's writeout from then on
      hipMemset(ws.slots, 0, DOMINO_T * Bm * kSlotSpan * 8) != hipSuccess ||
      hipMemset(ws.bad, 0, Bm * 4) != hipSuccess ||
      hipMemset(ws.hist, 0, Bm * 3 * 2048 * 4) != hipSuccess ||
      hipMemset(ws.base, 0, DOMINO_T * Bm * V * 4) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    set_global_err("create: workspace initialisation failed");
    domino_rollout_destroy(h);
    return DOMINO_ERR_HIP;
  }
  static std::once_flag once;
  std::call_once(once, [] {
    rowstream_prepare();
    lmhead_fused_prepare();
    lmhead_one_prepare();
    step_prepare();
  });
  // GRU input projection of every id, G[v, :] = W_ih E[v], the stacked step
  // weights in fragment order and fc2 in tile order; the weights are borrowed
  // and must not change for the handle's life
  launch_gru_table(h->shape, h->w, ws.G, nullptr);
  if (h->shape.bf16) launch_pack_step_weights(h->shape, h->w, ws.Wp, nullptr);
  if (ws.fc2p) launch_pack_tiles((const uint16_t*)h->w.fc2, (int)V, (int)r, ws.fc2p, nullptr);
  if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    set_global_err("create: building the GRU input-projection table failed");
    domino_rollout_destroy(h);
    return DOMINO_ERR_HIP;
  }
  *out = h;
  return DOMINO_OK;
}

// Destroys every cached graph (the device has finished their launches: the
// callers synchronise first, or the handle is going away with its work done).
static void drop_graphs(domino_rollout_t* h) {
  for (auto& g : h->graphs) {
    (void)hipGraphExecDestroy(g.exec);
    if (g.done) (void)hipEventDestroy(g.done);
  }
  h->graphs.clear();
}

extern "C" void domino_rollout_destroy(domino_rollout_t* h) {
  if (!h) return;
  for (auto& p : h->pending) {
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
  }
  for (auto e : h->free_events) (void)hipEventDestroy(e);
  drop_graphs(h);
  if (h->capture_stream) (void)hipStreamDestroy(h->capture_stream);
  for (void* p : h->allocations) (void)hipFree(p);
  delete h;
}

extern "C" const char* domino_rollout_last_error(const domino_rollout_t* h) {
  if (h) return h->err.c_str();
  std::lock_guard<std::mutex> lk(g_err_mu);
  static thread_local std::string copy;
  copy = g_err;
  return copy.c_str();
}

// Host-side checks only: nothing is read from the device.
static domino_status_t check_run_args(domino_rollout_t* h, const void* hidden, const float* s,
                                      const int32_t* ver, int32_t B, int32_t K, int32_t* out_tokens) {
  if (!h) return DOMINO_ERR_INVALID_ARG;
  if (!hidden || !ver || !out_tokens)
    return h->fail(DOMINO_ERR_INVALID_ARG, "run: hidden, verified_tokens and out_tokens must be non-NULL");
  if (!s && !h->w.fc1_x)
    return h->fail(DOMINO_ERR_INVALID_ARG,
                   "run: step_s is NULL and the handle holds no fc1_x_w / fc1_b to form it");
  if ((uintptr_t)hidden & 15)
    return h->fail(DOMINO_ERR_INVALID_ARG, "run: base_hidden must be 16-byte aligned");
  if ((uintptr_t)s & 3) return h->fail(DOMINO_ERR_INVALID_ARG, "run: step_s must be 4-byte aligned");
  if (B < 1 || B > h->cfg.max_batch)
    return h->fail(DOMINO_ERR_INVALID_ARG, "run: batch %d outside [1, %d]", B, h->cfg.max_batch);
  if (K < 0) return h->fail(DOMINO_ERR_INVALID_ARG, "run: K must be >= 0 (got %d)", K);
  if (K > 0 && K < h->cfg.vocab && K > h->cfg.max_k)
    return h->fail(DOMINO_ERR_INVALID_ARG, "run: pool size K=%d exceeds max_k=%d", K, h->cfg.max_k);
  return DOMINO_OK;
}

// Times the launches issued inside its scope: each kernel launched while it
// is active carries an event pair stamped by its own dispatch (see DLAUNCH),
// and the phase accumulates the kernels' durations.
namespace {
struct ActivePhase {
  domino_rollout_t* h;
  int phase;
};
thread_local ActivePhase* g_active_phase = nullptr;
}  // namespace

bool timing_events(hipEvent_t* start, hipEvent_t* stop) {
  ActivePhase* p = g_active_phase;
  if (!p) return false;
  hipEvent_t a = p->h->take_event(), b = p->h->take_event();
  if (!a || !b) {
    if (a) p->h->free_events.push_back(a);
    if (b) p->h->free_events.push_back(b);
    return false;
  }
  p->h->pending.push_back({p->phase, a, b});
  *start = a;
  *stop = b;
  return true;
}

struct PhaseTimer {
  domino_rollout_t* h;
  ActivePhase self;
  ActivePhase* prev = nullptr;
  bool on = false;
  PhaseTimer(domino_rollout_t* h_, int phase, hipStream_t) : h(h_), self{h_, phase} {
    if (h->timing && !h->capturing) {
      prev = g_active_phase;
      g_active_phase = &self;
      on = true;
    }
  }
  ~PhaseTimer() {
    if (!on) return;
    g_active_phase = prev;
    h->phase_n[self.phase] += 1;
  }
};

// One rollout producing the first P proposals (P = DOMINO_T: the whole block):
// base logits, first proposal and pool of the whole block, then P - 1
// correction steps.
static void enqueue(domino_rollout_t* h, const Workspace& ws, const void* hidden, const float* s,
                    const int32_t* ver, const int32_t* forced, int B, int K, int P,
                    int32_t* out_tokens, float* out_top1, hipStream_t st) {
  const Shape& sh = h->shape;
  const bool pool = K > 0 && K < sh.V;
  h->last_B = B;
  h->last_K = pool ? K : 0;
  h->last_union = pool && pool_union(sh, ws, B, K);
  h->last_s_internal = s == nullptr;
  if (!s) {
    // step offsets from the block's hiddens (projector layer 1, backbone half)
    PhaseTimer t(h, kOffsets, st);
    launch_step_offsets(sh, h->w, hidden, ws, B, st);
    s = ws.s;
  }
  const bool fused = sh.bf16 && B >= kFusedMinBatch && lmhead_fused_supported(sh.H);
  const bool one = sh.bf16 && B == 1 && lmhead_one_supported(sh.V, sh.H);
  if (one) {
    // base logits, pool-score keys and the first proposal in one pass
    PhaseTimer t(h, kLmHead, st);
    launch_lmhead_one((const uint16_t*)h->w.lm_head, (const uint16_t*)hidden, ws.base,
                      pool ? ws.keys : nullptr, pool ? ws.hist : nullptr, ws.slots, sh.V, sh.H,
                      st);
  } else if (fused) {
    // base logits, pool-score keys and the first proposal in one pass
    PhaseTimer t(h, kLmHead, st);
    FusedArgs fa{(const uint16_t*)h->w.lm_head, (const uint16_t*)hidden, ws.base,
                 pool ? ws.keys : nullptr, ws.slots, sh.V, sh.H, B, ws.xp};
    launch_lmhead_fused(fa, st);
  } else {
    {
      PhaseTimer t(h, kLmHead, st);
      launch_lmhead(sh, h->w.lm_head, hidden, ws.base, B, st);
    }
    PhaseTimer t(h, kArgmax0, st);
    launch_row0_argmax(sh, ws.base, B, ws.slots, st);
  }
  if (pool) {
    PhaseTimer t(h, kPool, st);
    launch_pool_build(sh, ws, h->w.fc2_b, B, K, fused || one, one, st);
  }
  // Prefix: h(1) = GRU(E[verified], 0) and c(1) = W_hh h(1).  It runs for
  // every P: its gates are where an invalid verified token is flagged.
  const int steps = P - 1;  // correction steps of this run
  const int path = step_path(sh, B, h->step_path);
  StepArgs sa{};
  sa.F1 = h->w.fc1;
  sa.W_hh = h->w.w_hh;
  sa.G = ws.G;
  sa.bad = ws.bad;
  sa.s = s;
  sa.u = ws.u;
  sa.u_hi = ws.u_hi;
  sa.u_lo = ws.u_lo;
  sa.partial = ws.partial;
  sa.Wp = ws.Wp;
  sa.hp = path == kStepMfma ? ws.hp : nullptr;  // only the matrix-core product reads it
  sa.B = B;
  sa.V = sh.V;
  sa.g = sh.g;
  sa.r = sh.r;
  auto step_launches = [&](int phase_gates, int phase_product) {
    if (path != kStepFused || sa.nrows == 0) {
      PhaseTimer t(h, phase_gates, st);
      launch_gru_gates(sa, st);
    }
    if (sa.nrows > 0) {
      PhaseTimer t(h, phase_product, st);
      launch_step_product(sh, sa, path, st);
    }
  };
  sa.h_prev = nullptr;
  sa.c_prev = nullptr;
  sa.h_new = ws.h[0];
  sa.c_new = ws.c[0];
  sa.tok_i32 = ver;
  sa.tok_stride = 1;
  sa.tok_key = nullptr;
  sa.row0 = sh.r;  // W_hh rows only
  sa.nrows = steps > 0 ? 3 * sh.g : 0;
  step_launches(kGru, kGru);
  int cur = 0;
  for (int k = 1; k <= steps; ++k) {
    // h(k+1) = GRU(E[p_k], h(k)); u = SiLU(fc1 h(k+1) + s[k-1]); c(k+1) = W_hh h(k+1)
    sa.h_prev = ws.h[cur];
    sa.c_prev = ws.c[cur];
    sa.h_new = ws.h[cur ^ 1];
    sa.c_new = ws.c[cur ^ 1];
    if (forced) {
      sa.tok_i32 = forced + (k - 1);
      sa.tok_stride = DOMINO_T;
      sa.tok_key = nullptr;
    } else {
      sa.tok_i32 = nullptr;
      sa.tok_key = ws.slots + (size_t)(k - 1) * B * kSlotSpan;
    }
    sa.step = k - 1;
    sa.row0 = 0;
    sa.nrows = k < steps ? sh.r + 3 * sh.g : sh.r;  // no W_hh after the last step
    step_launches(kGru, kStep);
    cur ^= 1;
    {
      PhaseTimer t(h, kCorrect, st);
      if (pool)
        launch_correct_pool(sh, h->w, ws, k, B, K, st);
      else
        launch_correct_full(sh, h->w, ws, k, B, st);
    }
  }
  launch_writeout(ws, B, P, pool, out_tokens, out_top1, st);
}

namespace {
struct DeviceGuard {
  int prev = -1, want;
  explicit DeviceGuard(int d) : want(d) {
    if (hipGetDevice(&prev) == hipSuccess && prev != want) (void)hipSetDevice(want);
  }
  ~DeviceGuard() {
    if (prev >= 0 && prev != want) (void)hipSetDevice(prev);
  }
};
}  // namespace

static domino_status_t run_common(domino_rollout_t* h, const void* hidden, const float* s,
                                  const int32_t* ver, const int32_t* forced, int32_t B, int32_t K,
                                  int32_t P, int32_t* out_tokens, float* out_top1, void* stream) {
  domino_status_t st = check_run_args(h, hidden, s, ver, B, K, out_tokens);
  if (st != DOMINO_OK) return st;
  DeviceGuard dg(h->device);
  (void)hipGetLastError();  // clear a stale error of an unrelated call
  enqueue(h, h->ws, hidden, s, ver, forced, B, K, P, out_tokens, out_top1, (hipStream_t)stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return h->fail(DOMINO_ERR_HIP, "run: kernel launch failed: %s", hipGetErrorString(e));
  h->err.clear();
  return DOMINO_OK;
}

extern "C" domino_status_t domino_rollout_run(domino_rollout_t* h, const void* base_hidden,
                                              const float* step_s, const int32_t* verified_tokens,
                                              int32_t batch, int32_t K, int32_t* out_tokens,
                                              float* out_top1_logit, void* stream) {
  return run_common(h, base_hidden, step_s, verified_tokens, nullptr, batch, K, DOMINO_T,
                    out_tokens, out_top1_logit, stream);
}

extern "C" domino_status_t domino_rollout_run_forced(domino_rollout_t* h, const void* base_hidden,
                                                     const float* step_s,
                                                     const int32_t* verified_tokens,
                                                     const int32_t* forced_tokens, int32_t batch,
                                                     int32_t K, int32_t* out_tokens,
                                                     float* out_top1_logit, void* stream) {
  if (h && !forced_tokens) return h->fail(DOMINO_ERR_INVALID_ARG, "run_forced: forced_tokens is NULL");
  return run_common(h, base_hidden, step_s, verified_tokens, forced_tokens, batch, K, DOMINO_T,
                    out_tokens, out_top1_logit, stream);
}

// Carves the per-run buffers of a B-request run out of `base` (256-byte
// aligned pieces) into ws and returns the bytes they take; with base ==
// nullptr only the size is computed.
static size_t carve_static(const domino_rollout_t* h, int B, Workspace& ws, unsigned char* base) {
  const Shape& sh = h->shape;
  const size_t g = sh.g, r = sh.r, Bz = B;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? (void*)(base + off) : nullptr;
    off += (bytes + 255) / 256 * 256;
    return p;
  };
  ws.slots = (uint64_t*)take(DOMINO_T * Bz * kSlotSpan * 8);
  ws.bad = (int32_t*)take(Bz * 4);
  ws.hist = (uint32_t*)take(Bz * 3 * 2048 * 4);
  ws.state = (uint32_t*)take(Bz * 8 * 4);
  ws.h[0] = (float*)take(Bz * g * 4);
  ws.h[1] = (float*)take(Bz * g * 4);
  ws.c[0] = (float*)take(Bz * 3 * g * 4);
  ws.c[1] = (float*)take(Bz * 3 * g * 4);
  ws.u = (float*)take(Bz * r * 4);
  ws.u_hi = (uint16_t*)take(Bz * r * 2);
  ws.u_lo = (uint16_t*)take(Bz * r * 2);
  ws.hp = sh.bf16 ? (uint16_t*)take((Bz + 15) / 16 * 16 * g * 4) : nullptr;
  ws.partial = (float*)take(step_partial_floats((int)g, (int)r) * sizeof(float));
  return off;
}

extern "C" domino_status_t domino_rollout_run_static(domino_rollout_t* h, const void* base_hidden,
                                                     const float* step_s,
                                                     const int32_t* verified_tokens, int32_t batch,
                                                     int32_t K, int32_t* out_tokens,
                                                     float* out_top1_logit, void* stream) {
  domino_status_t st = check_run_args(h, base_hidden, step_s, verified_tokens, batch, K, out_tokens);
  if (st != DOMINO_OK) return st;
  Workspace ws = h->ws;
  const size_t need = carve_static(h, batch, ws, nullptr);
  if (need > kStaticScratchBytes)
    return h->fail(DOMINO_ERR_INVALID_ARG,
                   "run_static: %d requests need %zu bytes of scratch, more than the %zu of the "
                   "static array", batch, need, kStaticScratchBytes);
  DeviceGuard dg(h->device);
  unsigned char* base = (unsigned char*)static_scratch(h->device);
  if (!base) return h->fail(DOMINO_ERR_UNSUPPORTED, "run_static: no static scratch on this device");
  carve_static(h, batch, ws, base);
  (void)hipGetLastError();
  // the argmax words, flags and histograms must start at zero, whatever an
  // earlier call on this device left (a fill kernel, so the call can be captured)
  const size_t n16 = need / 16;
  hipLaunchKernelGGL(scratch_clear_kernel, dim3((unsigned)std::min<size_t>((n16 + 255) / 256, 1024)),
                     dim3(256), 0, (hipStream_t)stream, (uint4*)base, n16);
  enqueue(h, ws, base_hidden, step_s, verified_tokens, nullptr, batch, K, DOMINO_T, out_tokens,
          out_top1_logit, (hipStream_t)stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return h->fail(DOMINO_ERR_HIP, "run_static: kernel launch failed: %s", hipGetErrorString(e));
  h->err.clear();
  return DOMINO_OK;
}

static domino_status_t run_graph_common(domino_rollout_t* h, const void* base_hidden,
                                        const float* step_s, const int32_t* verified_tokens,
                                        int32_t batch, int32_t K, int32_t P, int32_t* out_tokens,
                                        float* out_top1_logit, void* stream) {
  domino_status_t st = check_run_args(h, base_hidden, step_s, verified_tokens, batch, K, out_tokens);
  if (st != DOMINO_OK) return st;
  DeviceGuard dg(h->device);
  const int kmode = (K > 0 && K < h->cfg.vocab) ? K : 0;
  GraphKey key{batch, kmode, 0, P,
               {base_hidden, step_s, verified_tokens, out_tokens, out_top1_logit, nullptr}};
  GraphEntry* ent = nullptr;
  for (auto& g : h->graphs)
    if (g.key == key) ent = &g;
  if (!ent) {
    if (h->graphs.size() >= DOMINO_GRAPH_CACHE_MAX) {
      // evict the least recently used graph once its last replay has ended
      auto lru = std::min_element(h->graphs.begin(), h->graphs.end(),
                                  [](const GraphEntry& a, const GraphEntry& b) { return a.used < b.used; });
      if (hipEventSynchronize(lru->done) != hipSuccess)
        return h->fail(DOMINO_ERR_HIP, "run_graph: waiting for an evicted graph failed");
      (void)hipGraphExecDestroy(lru->exec);
      (void)hipEventDestroy(lru->done);
      h->graphs.erase(lru);
    }
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;
    if (hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess)
      return h->fail(DOMINO_ERR_HIP, "run_graph: event creation failed");
    if (!h->capture_stream &&
        hipStreamCreateWithFlags(&h->capture_stream, hipStreamNonBlocking) != hipSuccess)
      return h->fail(DOMINO_ERR_HIP, "run_graph: stream creation failed");
    (void)hipGetLastError();
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(h->capture_stream, hipStreamCaptureModeRelaxed) != hipSuccess) {
      (void)hipEventDestroy(done);
      return h->fail(DOMINO_ERR_HIP, "run_graph: begin capture failed");
    }
    h->capturing = true;
    enqueue(h, h->ws, base_hidden, step_s, verified_tokens, nullptr, batch, kmode, P, out_tokens,
            out_top1_logit, h->capture_stream);
    h->capturing = false;
    hipError_t e1 = hipGetLastError();
    hipError_t e2 = hipStreamEndCapture(h->capture_stream, &graph);
    if (e1 != hipSuccess || e2 != hipSuccess || !graph) {
      if (graph) (void)hipGraphDestroy(graph);
      (void)hipEventDestroy(done);
      return h->fail(DOMINO_ERR_HIP, "run_graph: capture failed: %s",
                     hipGetErrorString(e1 != hipSuccess ? e1 : e2));
    }
    hipError_t e3 = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e3 != hipSuccess) {
      (void)hipEventDestroy(done);
      return h->fail(DOMINO_ERR_HIP, "run_graph: instantiate failed: %s", hipGetErrorString(e3));
    }
    h->graphs.push_back(GraphEntry{key, exec, done, 0, h->last_B, h->last_K, h->last_union,
                                   h->last_s_internal});
    ent = &h->graphs.back();
  }
  ent->used = ++h->graph_clock;
  // the workspace now holds this graph's run
  h->last_B = ent->last_B;
  h->last_K = ent->last_K;
  h->last_union = ent->last_union;
  h->last_s_internal = ent->last_s_internal;
  hipError_t e = hipGraphLaunch(ent->exec, (hipStream_t)stream);
  if (e != hipSuccess) return h->fail(DOMINO_ERR_HIP, "run_graph: launch failed: %s", hipGetErrorString(e));
  if (hipEventRecord(ent->done, (hipStream_t)stream) != hipSuccess)
    return h->fail(DOMINO_ERR_HIP, "run_graph: event record failed");
  h->err.clear();
  return DOMINO_OK;
}

extern "C" domino_status_t domino_rollout_cached_graphs(const domino_rollout_t* h, int32_t* count) {
  if (!h || !count) return DOMINO_ERR_INVALID_ARG;
  *count = (int32_t)h->graphs.size();
  return DOMINO_OK;
}

extern "C" domino_status_t domino_rollout_run_graph(domino_rollout_t* h, const void* base_hidden,
                                                    const float* step_s,
                                                    const int32_t* verified_tokens, int32_t batch,
                                                    int32_t K, int32_t* out_tokens,
                                                    float* out_top1_logit, void* stream) {
  return run_graph_common(h, base_hidden, step_s, verified_tokens, batch, K, DOMINO_T, out_tokens,
                          out_top1_logit, stream);
}

extern "C" domino_status_t domino_rollout_run_prefix(domino_rollout_t* h, const void* base_hidden,
                                                     const float* step_s,
                                                     const int32_t* verified_tokens, int32_t batch,
                                                     int32_t K, int32_t proposals,
                                                     int32_t* out_tokens, float* out_top1_logit,
                                                     int32_t graph, void* stream) {
  if (!h) return DOMINO_ERR_INVALID_ARG;
  if (proposals < 1 || proposals > DOMINO_T)
    return h->fail(DOMINO_ERR_INVALID_ARG, "run_prefix: proposals %d outside [1, %d]", proposals,
                   DOMINO_T);
  if (graph)
    return run_graph_common(h, base_hidden, step_s, verified_tokens, batch, K, proposals,
                            out_tokens, out_top1_logit, stream);
  return run_common(h, base_hidden, step_s, verified_tokens, nullptr, batch, K, proposals,
                    out_tokens, out_top1_logit, stream);
}

extern "C" domino_status_t domino_rollout_read_workspace(const domino_rollout_t* h, int32_t which,
                                                         void* dst, size_t dst_bytes, size_t* bytes,
                                                         void* stream) {
  if (!h || !bytes || h->last_B <= 0) return DOMINO_ERR_INVALID_ARG;
  const void* src = nullptr;
  size_t n = 0;
  if (which == 0) {
    src = h->ws.base;
    n = (size_t)DOMINO_T * h->last_B * h->cfg.vocab * 4;
  } else if (which == 1 && h->last_K > 0) {
    src = h->ws.pool_ids;
    n = (size_t)h->last_B * h->last_K * 4;
  } else if (which == 2 && h->last_s_internal) {
    src = h->ws.s;
    n = (size_t)h->last_B * DOMINO_S * h->cfg.proj_dim * 4;
  } else if (which == 3 && h->last_union) {
    src = h->ws.un;
    n = (size_t)((h->last_B + h->ws.ugroup - 1) / h->ws.ugroup) * 4;
  } else {
    return DOMINO_ERR_INVALID_ARG;
  }
  *bytes = n;
  if (!dst) return DOMINO_OK;
  if (dst_bytes < n) return DOMINO_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  if (hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, (hipStream_t)stream) != hipSuccess)
    return DOMINO_ERR_HIP;
  return DOMINO_OK;
}

extern "C" domino_status_t domino_rollout_set_pool_strategy(domino_rollout_t* h,
                                                            int32_t strategy) {
  if (!h) return DOMINO_ERR_INVALID_ARG;
  if (strategy < 0 || strategy > 2)
    return h->fail(DOMINO_ERR_INVALID_ARG, "set_pool_strategy: strategy must be 0, 1 or 2");
  if (strategy != h->ws.pool_strategy) {
    DeviceGuard dg(h->device);
    if (hipDeviceSynchronize() != hipSuccess)
      return h->fail(DOMINO_ERR_HIP, "set_pool_strategy: synchronize failed");
    drop_graphs(h);  // captured the old strategy
    h->ws.pool_strategy = strategy;
  }
  return DOMINO_OK;
}

extern "C" domino_status_t domino_rollout_set_step_path(domino_rollout_t* h, int32_t path) {
  if (!h) return DOMINO_ERR_INVALID_ARG;
  if (path < kStepAuto || path > kStepMfma)
    return h->fail(DOMINO_ERR_INVALID_ARG, "set_step_path: path must be 0, 1, 2 or 3");
  if (path != h->step_path) {
    DeviceGuard dg(h->device);
    if (hipDeviceSynchronize() != hipSuccess)
      return h->fail(DOMINO_ERR_HIP, "set_step_path: synchronize failed");
    drop_graphs(h);  // captured the old path
    h->step_path = path;
  }
  return DOMINO_OK;
}

extern "C" domino_status_t domino_rollout_set_timing(domino_rollout_t* h, int32_t enable) {
  if (!h) return DOMINO_ERR_INVALID_ARG;
  h->timing = enable != 0;
  return DOMINO_OK;
}

extern "C" domino_status_t domino_rollout_kernel_times(domino_rollout_t* h, int32_t which,
                                                       double* total_ms, int64_t* launches) {
  if (!h || which < -1 || which >= kPhases) return DOMINO_ERR_INVALID_ARG;
  DeviceGuard dg(h->device);
  for (auto& p : h->pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess)
      return h->fail(DOMINO_ERR_HIP, "kernel_times: event query failed");
    h->phase_ms[p.phase] += ms;
    h->free_events.push_back(p.a);
    h->free_events.push_back(p.b);
  }
  h->pending.clear();
  if (which == -1) {
    for (int i = 0; i < kPhases; ++i) {
      h->phase_ms[i] = 0;
      h->phase_n[i] = 0;
    }
    return DOMINO_OK;
  }
  if (total_ms) *total_ms = h->phase_ms[which];
  if (launches) *launches = h->phase_n[which];
  return DOMINO_OK;
}
