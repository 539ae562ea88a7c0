// Step kernels of the Domino draft-block rollout for gfx950.
//
// Method (cited by page title and section):
//  * "Add correctness-first Domino support to DFlash V2" (sglang PR #31328),
//    "Design": first proposal = full-vocabulary argmax of the base logits;
//    bias-free GRU over [verified, first proposal]; one block-shared pool of
//    K ids per request (K = 0: full vocabulary); each realised proposal is
//    fed back before the next correction step.
//  * "[Spec] Add Domino projector support to DFlash speculative decoding
//    (V2)" (sglang PR #28998), "Implementation": fused SiLU(z+s)·fc2ᵀ + bias +
//    base_logits followed by the argmax; a fused GRU cell.
//  * "feat: support tensor-parallel Domino rollout" (sglang PR #32018),
//    "Implementation" / "Validation and limitations": the pool is a TopK of
//    the block's base logits whose cutoff ties the page leaves open (here:
//    lower id wins).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

#include "frag.h"

// ------------------------------------------------ per-step projector offsets
// step_s[b, j, n] = fc1_x[n, :] . X[b, j+1, :] + fc1_b[n], j = 0..13: the
// backbone-hidden half of the projector's first layer ([backbone hidden |
// GRU state], "Add correctness-first Domino support to DFlash V2", commit
// text) and its bias, for the hidden of the position whose base row the
// correction step scores.
//
// bf16 models: one MFMA product C[m, n] over the M = 14B (request, step) rows
// m = 14b + j, which is exactly the row order of step_s, so the epilogue
// stores straight into [B, 14, r].  A workgroup computes 64 units n x 64 rows
// m; its four waves own 32 x 32 each (2 x 2 tiles of 16x16x32).  k runs in
// slices of 64 staged in LDS (two buffers, rows padded to 144 bytes so the
// fragment reads of 16 lanes hit distinct banks), fed from four register
// stages so each slice's 16-byte loads have three steps to land.  With
// fewer tiles than CUs (small batches) k is split over workgroups until
// about one per CU, each writing its partial product, and a combine kernel
// adds the splits in a fixed order and the bias.  fp32 models (small) take a
// direct kernel.
//
// The same product forms the GRU input-projection table G[v, :] = W_ih E[v]
// when a handle is created: row m of the activations is then simply E[m]
// (the row map below with one row per group), the units are W_ih's 3g rows
// and there is no bias.
constexpr int kOfsTile = 64;           // units and rows per workgroup
constexpr int kOfsSlice = 64;          // k per LDS stage
constexpr int kOfsPitch = 72;          // LDS row pitch in bf16 (144 bytes)
constexpr int kOfsMinSlices = 4;       // k slices per split at least
constexpr int kOfsTargetGroups = 256;  // split k until about this many workgroups

// one 64-wide k slice of a wave's 32 x 32 block from LDS buffers lw / lx
__device__ __forceinline__ void offsets_mma(const bf16_t* lw, const bf16_t* lx, int wn, int wm,
                                            int fr, int fq, v4f (&acc)[2][2]) {
#pragma unroll
  for (int ks = 0; ks < kOfsSlice / 32; ++ks) {
    const int c = ks * 32 + 8 * fq;
    const v8s a0 = *reinterpret_cast<const v8s*>(lw + (32 * wn + fr) * kOfsPitch + c);
    const v8s a1 = *reinterpret_cast<const v8s*>(lw + (32 * wn + 16 + fr) * kOfsPitch + c);
    const v8s b0 = *reinterpret_cast<const v8s*>(lx + (32 * wm + fr) * kOfsPitch + c);
    const v8s b1 = *reinterpret_cast<const v8s*>(lx + (32 * wm + 16 + fr) * kOfsPitch + c);
    acc[0][0] = mfma_bf16(a0, b0, acc[0][0]);
    acc[0][1] = mfma_bf16(a0, b1, acc[0][1]);
    acc[1][0] = mfma_bf16(a1, b0, acc[1][0]);
    acc[1][1] = mfma_bf16(a1, b1, acc[1][1]);
  }
}

__global__ __launch_bounds__(256) void offsets_gemm_kernel(const bf16_t* __restrict__ W,
                                                           const bf16_t* __restrict__ X,
                                                           const bf16_t* __restrict__ b1,
                                                           float* __restrict__ out, int M, int N,
                                                           int H, int kper, int rpg, int gstride,
                                                           int roff) {
  __shared__ __attribute__((aligned(16))) bf16_t lw[2][kOfsTile * kOfsPitch];
  __shared__ __attribute__((aligned(16))) bf16_t lx[2][kOfsTile * kOfsPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int n0 = blockIdx.x * kOfsTile, m0 = blockIdx.y * kOfsTile, split = blockIdx.z;
  const int kbeg = split * kper, nsl = kper / kOfsSlice;
  // loader: thread t moves 16 bytes at column 8 (t % 8) of rows t / 8 and t / 8 + 32
  // (rows past the end are clamped: loaded and dropped).  Activation row m is
  // row (m / rpg) * gstride + m % rpg + roff of X (step offsets: the hiddens
  // of positions 1..14 of each request; the G table: E row m).  b1 may be NULL.
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const int na = min(n0 + lr, N - 1), nb = min(n0 + lr + 32, N - 1);
  const int ma = min(m0 + lr, M - 1), mb = min(m0 + lr + 32, M - 1);
  const bf16_t* wpa = W + (size_t)na * H + kbeg + lc;
  const bf16_t* wpb = W + (size_t)nb * H + kbeg + lc;
  const bf16_t* xpa = X + ((size_t)(ma / rpg) * gstride + ma % rpg + roff) * H + kbeg + lc;
  const bf16_t* xpb = X + ((size_t)(mb / rpg) * gstride + mb % rpg + roff) * H + kbeg + lc;
  const int sta = lr * kOfsPitch + lc, stb = (lr + 32) * kOfsPitch + lc;
  // four register stages (named, so they stay in registers): slice k is
  // fetched into stage k % 4 three steps before it is put into LDS buffer
  // k % 2, at the end of the step that multiplies slice k - 1
  uint4 w0a, w0b, x0a, x0b, w1a, w1b, x1a, x1b, w2a, w2b, x2a, x2b, w3a, w3b, x3a, x3b;
#define OFS_FETCH(S, SL)                                           \
  do {                                                             \
    const size_t o_ = (size_t)min(SL, nsl - 1) * kOfsSlice;        \
    w##S##a = *reinterpret_cast<const uint4*>(wpa + o_);           \
    w##S##b = *reinterpret_cast<const uint4*>(wpb + o_);           \
    x##S##a = *reinterpret_cast<const uint4*>(xpa + o_);           \
    x##S##b = *reinterpret_cast<const uint4*>(xpb + o_);           \
  } while (0)
#define OFS_PUT(BUF, S)                                            \
  do {                                                             \
    *reinterpret_cast<uint4*>(&lw[BUF][sta]) = w##S##a;            \
    *reinterpret_cast<uint4*>(&lw[BUF][stb]) = w##S##b;            \
    *reinterpret_cast<uint4*>(&lx[BUF][sta]) = x##S##a;            \
    *reinterpret_cast<uint4*>(&lx[BUF][stb]) = x##S##b;            \
  } while (0)
  // step h (stage j = h % 4): fetch slice h + 3, multiply slice h from
  // buffer h % 2, put slice h + 1 into the other buffer (last read before
  // the previous barrier).  Slices past the end are clamped to the last one
  // (loaded, never multiplied).
#define OFS_STEP(H, FETCH_S, BUF, PUT_S)                            \
  do {                                                             \
    OFS_FETCH(FETCH_S, (H) + 3);                                   \
    __builtin_amdgcn_sched_barrier(0);                             \
    offsets_mma(lw[BUF], lx[BUF], wn, wm, fr, fq, acc);            \
    OFS_PUT(BUF ^ 1, PUT_S);                                       \
    __syncthreads();                                               \
  } while (0)
  const int wn = wave & 1, wm = wave >> 1, fr = lane & 15, fq = lane >> 4;
  v4f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = v4f{0.f, 0.f, 0.f, 0.f};
  OFS_FETCH(0, 0);
  OFS_FETCH(1, 1);
  OFS_FETCH(2, 2);
  OFS_PUT(0, 0);
  __syncthreads();
  int h = 0;
  for (; h + 4 <= nsl; h += 4) {
    OFS_STEP(h, 3, 0, 1);
    OFS_STEP(h + 1, 0, 1, 2);
    OFS_STEP(h + 2, 1, 0, 3);
    OFS_STEP(h + 3, 2, 1, 0);
  }
  if (h < nsl) OFS_STEP(h, 3, 0, 1);
  if (h + 1 < nsl) OFS_STEP(h + 1, 0, 1, 2);
  if (h + 2 < nsl) OFS_STEP(h + 2, 1, 0, 3);
#undef OFS_STEP
#undef OFS_FETCH
#undef OFS_PUT
  // lane: row m = m0 + 32 wm + 16 jj + fr, units n = n0 + 32 wn + 16 i + 4 fq + 0..3
  const bool whole = gridDim.z == 1;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = n0 + 32 * wn + 16 * i + 4 * fq;
    if (n >= N) continue;  // N % 4 == 0, so n < N covers n + 3
    float bias[4] = {0.f, 0.f, 0.f, 0.f};
    if (whole && b1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) bias[c] = bf16_to_f32(b1[n + c]);
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int m = m0 + 32 * wm + 16 * jj + fr;
      if (m >= M) continue;
      float* o = out + ((size_t)split * M + m) * N + n;
      *reinterpret_cast<float4*>(o) = make_float4(acc[i][jj][0] + bias[0], acc[i][jj][1] + bias[1],
                                                  acc[i][jj][2] + bias[2], acc[i][jj][3] + bias[3]);
    }
  }
}

// s = sum of the split partials in split order, plus the bias
__global__ __launch_bounds__(256) void offsets_combine_kernel(const float* __restrict__ part,
                                                              const bf16_t* __restrict__ b1,
                                                              float* __restrict__ s, int M, int N,
                                                              int splits) {
  const int idx = blockIdx.x * 256 + threadIdx.x;  // one float4 of s
  const size_t MN = (size_t)M * N;
  if ((size_t)idx * 4 >= MN) return;
  const int n = (int)(((size_t)idx * 4) % N);
  float4 acc = reinterpret_cast<const float4*>(part)[idx];
  for (int p = 1; p < splits; ++p) {
    const float4 v = reinterpret_cast<const float4*>(part + p * MN)[idx];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  acc.x += bf16_to_f32(b1[n]);
  acc.y += bf16_to_f32(b1[n + 1]);
  acc.z += bf16_to_f32(b1[n + 2]);
  acc.w += bf16_to_f32(b1[n + 3]);
  reinterpret_cast<float4*>(s)[idx] = acc;
}

// fp32 models: one thread per entry of s
__global__ __launch_bounds__(256) void step_offsets_f32_kernel(const float* __restrict__ X,
                                                               const float* __restrict__ W,
                                                               const float* __restrict__ b1,
                                                               float* __restrict__ s, int B, int H,
                                                               int r) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= B * DOMINO_S * r) return;
  const int b = idx / (DOMINO_S * r), rem = idx - b * (DOMINO_S * r);
  const int j = rem / r, n = rem - j * r;
  const float* x = X + ((size_t)b * DOMINO_T + j + 1) * H;
  const float* wr = W + (size_t)n * H;
  float acc = 0.f;
  for (int i = 0; i < H; ++i) acc = fmaf(x[i], wr[i], acc);
  s[idx] = acc + b1[n];
}

// k splits of the offsets product for a batch of B (1 when it is not tiled)
int step_offsets_splits(int B, int H, int r) {
  if (H % kOfsSlice != 0 || r % 4 != 0) return 1;
  const int tiles = ((r + kOfsTile - 1) / kOfsTile) * ((B * DOMINO_S + kOfsTile - 1) / kOfsTile);
  const int nsl = H / kOfsSlice;
  int splits = 1;
  while (splits * 2 * tiles <= kOfsTargetGroups && nsl % (splits * 2) == 0 &&
         nsl / (splits * 2) >= kOfsMinSlices)
    splits *= 2;
  return splits;
}

size_t step_offsets_partial_floats(int Bmax, int H, int r) {
  size_t most = 0;
  for (int B = 1; B <= Bmax; ++B) {
    const int sp = step_offsets_splits(B, H, r);
    if (sp > 1) most = std::max(most, (size_t)sp * B * DOMINO_S * r);
  }
  return most;
}

void launch_step_offsets(const Shape& s, const DeviceWeights& w, const void* X, const Workspace& ws,
                         int B, hipStream_t st) {
  const int M = B * DOMINO_S, N = s.r, H = s.H, n = M * N;
  if (s.bf16) {  // create() and run() guarantee H % 64 == 0, r % 32 == 0, 16-byte aligned rows
    const int splits = step_offsets_splits(B, H, N);
    const dim3 grid((N + kOfsTile - 1) / kOfsTile, (M + kOfsTile - 1) / kOfsTile, splits);
    DLAUNCH(offsets_gemm_kernel, grid, dim3(256), 0, st, (const bf16_t*)w.fc1_x,
            (const bf16_t*)X, (const bf16_t*)w.fc1_b, splits > 1 ? ws.s_tmp : ws.s, M, N, H,
            H / splits, DOMINO_S, DOMINO_T, 1);
    if (splits > 1)
      DLAUNCH(offsets_combine_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, st,
              (const float*)ws.s_tmp, (const bf16_t*)w.fc1_b, ws.s, M, N, splits);
  } else {
    DLAUNCH(step_offsets_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, (const float*)X,
            (const float*)w.fc1_x, (const float*)w.fc1_b, ws.s, B, H, N);
  }
}

// ------------------------------------------------ GRU input-projection table
// G[v, n] = sum_i W_ih[n, i] E[v, i] for every vocabulary id v and gate row n
// (3g rows ordered r, z, n), fp32.  Formed once per handle; a GRU update of
// token x then reads row G[x] instead of multiplying W_ih by E[x].
template <bool BF>
__global__ __launch_bounds__(256) void gru_table_direct_kernel(const W_t<BF>* __restrict__ E,
                                                               const W_t<BF>* __restrict__ w_ih,
                                                               float* __restrict__ G, int V, int n3,
                                                               int e) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)V * n3) return;
  const int v = (int)(idx / n3), n = (int)(idx - (size_t)v * n3);
  const W_t<BF>* x = E + (size_t)v * e;
  const W_t<BF>* wr = w_ih + (size_t)n * e;
  float acc = 0.f;
  for (int i = 0; i < e; ++i) acc = fmaf(load_w<BF>(x + i), load_w<BF>(wr + i), acc);
  G[idx] = acc;
}

void launch_gru_table(const Shape& s, const DeviceWeights& w, float* G, hipStream_t st) {
  const int n3 = 3 * s.g;
  if (s.bf16 && s.e % kOfsSlice == 0) {
    // 64 x 64 tiles; units (W_ih rows) fastest, so the W_ih panel stays in L2
    const dim3 grid((n3 + kOfsTile - 1) / kOfsTile, (s.V + kOfsTile - 1) / kOfsTile, 1);
    hipLaunchKernelGGL(offsets_gemm_kernel, grid, dim3(256), 0, st, (const bf16_t*)w.w_ih,
                       (const bf16_t*)w.embed, (const bf16_t*)nullptr, G, s.V, n3, s.e, s.e, 1, 1,
                       0);
  } else {
    const size_t n = (size_t)s.V * n3;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (s.bf16)
      hipLaunchKernelGGL((gru_table_direct_kernel<true>), grid, dim3(256), 0, st,
                         (const bf16_t*)w.embed, (const bf16_t*)w.w_ih, G, s.V, n3, s.e);
    else
      hipLaunchKernelGGL((gru_table_direct_kernel<false>), grid, dim3(256), 0, st,
                         (const float*)w.embed, (const float*)w.w_ih, G, s.V, n3, s.e);
  }
}

// ---------------------------------------------------------------- reset
// There is no reset launch: a run's writeout (the last kernel of every run)
// clears the argmax words, the bad-token flags and the radix histograms it
// leaves behind, create() clears them once, and the first selection takes
// its initial state (empty prefix, rank K) from K itself.

// ------------------------------------------------------- first proposal (p1)
// argmax over the full vocabulary of base row 0 (t = 0), one argmax word per request
__global__ __launch_bounds__(256) void row0_argmax_kernel(const float* __restrict__ base, int V,
                                                          uint64_t* __restrict__ slots) {
  const int b = blockIdx.y;
  const float* row = base + (size_t)b * V;
  const int v_end = min(V, (int)(blockIdx.x + 1) * 2048);
  uint64_t best = 0;
  for (int v = blockIdx.x * 2048 + threadIdx.x; v < v_end; v += 256)
    best = umax64(best, pack_key(row[v], (uint32_t)v));
  best = wave_max_u64(best);
  __shared__ uint64_t wb[4];
  if ((threadIdx.x & 63) == 0) wb[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) publish_slot(slots, b, umax64(umax64(wb[0], wb[1]), umax64(wb[2], wb[3])));
}

void launch_row0_argmax(const Shape& s, const float* base, int B, uint64_t* slots, hipStream_t st) {
  DLAUNCH(row0_argmax_kernel, dim3((s.V + 2047) / 2048, B), dim3(256), 0, st, base, s.V,
                     slots);
}

// ---------------------------------------------------------------- pool build
// Radix select of the K largest per-id scores score[v] = max_t base[t,b,v]
// (as order-preserving uint32 keys) with 11 + 11 + 10 bit passes; the ids
// that can still be selected after two passes are collected, and the last
// pass and the compaction in id order (every key above the threshold and the
// lowest ids among keys equal to it) run over them alone.

__device__ __forceinline__ int block_excl_scan_256(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds[w] = x;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += lds[i];
  if (total) *total = lds[0] + lds[1] + lds[2] + lds[3];
  __syncthreads();
  return off + x - v;
}

__device__ __forceinline__ int block_sum_256(int v, int* lds) {
  int t;
  block_excl_scan_256(v, lds, &t);
  return t;
}

// The pool kernels take chunks of F * kPoolChunk ids per workgroup: larger
// chunks for larger batches, where the per-workgroup cost (clearing and
// flushing the bins, repeating the selection) would otherwise dominate.
template <int F>
__global__ __launch_bounds__(256) void pool_score_hist_kernel(const float* __restrict__ base, int V,
                                                              int B, uint32_t* __restrict__ keys,
                                                              uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[2048];
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < 2048; i += 256) h[i] = 0;
  __syncthreads();
  // every load is issued at a clamped address before any is used (a load
  // guarded by a divergent branch makes the compiler wait after each one)
  const int v0 = blockIdx.x * F * kPoolChunk;
#pragma unroll
  for (int j = 0; j < F * kPoolChunk / 256; ++j) {
    const int v = v0 + j * 256 + threadIdx.x;
    const int vc = min(v, V - 1);
    float x[DOMINO_T];
#pragma unroll
    for (int t = 0; t < DOMINO_T; ++t) x[t] = base[((size_t)t * B + b) * V + vc];
    float sc = x[0];
#pragma unroll
    for (int t = 1; t < DOMINO_T; ++t) sc = fmaxf(sc, x[t]);
    const uint32_t key = orderable(sc);
    if (v < V) {
      keys[(size_t)b * V + v] = key;
      atomicAdd(&h[key >> 21], 1u);
    }
  }
  __syncthreads();
  uint32_t* hh = hist + (size_t)b * 3 * 2048;
  for (int i = threadIdx.x; i < 2048; i += 256)
    if (h[i]) atomicAdd(&hh[i], h[i]);
}

// The radix state of request b after s selections sits at state[8 b + 2 s]
// (key prefix so far) and state[8 b + 2 s + 1] (rank of the K-th key among
// the keys with that prefix), s = 1, 2.  The state s = 0, (empty prefix, K),
// is never stored: the first selection (inside pool_hist_kernel<1>) starts
// from the kernel's K argument.

// Block-wide (256 threads): the bin of pass PASS (histogram hh) that holds
// the need-th largest key with the current prefix; returns the extended
// prefix and the rank left inside that bin.  Exactly one bin qualifies, so
// one thread writes res; every thread returns the result.
template <int PASS>
struct SelectBins {
  static constexpr int NBINS = PASS < 2 ? 2048 : 1024;
  static constexpr int PER = NBINS / 256;
  uint32_t c[PER];
  // thread 0 holds the highest PER bins, thread 255 the lowest
  __device__ __forceinline__ static int lo_bin() { return NBINS - ((int)threadIdx.x + 1) * PER; }
  __device__ __forceinline__ void load(const uint32_t* __restrict__ hh) {
#pragma unroll
    for (int j = 0; j < PER; ++j) c[j] = hh[lo_bin() + j];
  }
};

// the same with this thread's bins already loaded
template <int PASS>
__device__ __forceinline__ uint2 select_bin(const SelectBins<PASS>& bins, uint32_t prefix,
                                            uint32_t need, int* lds, uint32_t* res) {
  constexpr int PER = SelectBins<PASS>::PER;
  constexpr int BITS = PASS < 2 ? 11 : 10;
  const int lo_bin = SelectBins<PASS>::lo_bin();
  const uint32_t* const c = bins.c;
  int tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) tot += (int)c[j];
  uint32_t above = (uint32_t)block_excl_scan_256(tot, lds, nullptr);
#pragma unroll
  for (int j = PER - 1; j >= 0; --j) {
    if (above < need && above + c[j] >= need) {
      res[0] = (prefix << BITS) | (uint32_t)(lo_bin + j);
      res[1] = need - above;
    }
    above += c[j];
  }
  __syncthreads();
  return make_uint2(res[0], res[1]);
}

template <int PASS>
__device__ __forceinline__ uint2 select_bin(const uint32_t* __restrict__ hh, uint32_t prefix,
                                            uint32_t need, int* lds, uint32_t* res) {
  SelectBins<PASS> bins;
  bins.load(hh);
  return select_bin<PASS>(bins, prefix, need, lds, res);
}

// Histogram pass PASS (0 or 1) of the keys of request blockIdx.y in one
// chunk of ids.  Pass 1 first repeats the first selection in every workgroup
// (from its finished histogram) instead of in a launch of its own; the
// chunk-0 workgroup records the new state for the next kernel.
template <int PASS, int F>
__global__ __launch_bounds__(256) void pool_hist_kernel(const uint32_t* __restrict__ keys, int V,
                                                        uint32_t* __restrict__ state,
                                                        uint32_t* __restrict__ hist, int K) {
  static_assert(PASS == 0 || PASS == 1, "the last pass runs in pool_collect_kernel");
  constexpr int NBINS = 2048;
  __shared__ uint32_t h[NBINS];
  __shared__ int lds[4];
  __shared__ uint32_t res[2];
  const int b = blockIdx.y;
  // all key loads first, at clamped addresses (see pool_score_hist_kernel),
  // so they are in flight during the selection
  constexpr int NL = F * kPoolChunk / 256;
  const int v0 = blockIdx.x * F * kPoolChunk;
  uint32_t kv[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) kv[j] = keys[(size_t)b * V + min(v0 + j * 256 + (int)threadIdx.x, V - 1)];
  for (int i = threadIdx.x; i < NBINS; i += 256) h[i] = 0;
  uint32_t prefix = 0;
  if (PASS == 1) {
    // the state before the first selection is (empty prefix, rank K)
    const uint2 ns = select_bin<0>(hist + (size_t)b * 3 * 2048, 0u, (uint32_t)K, lds, res);
    prefix = ns.x;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      state[8 * b + 2] = ns.x;
      state[8 * b + 3] = ns.y;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const bool ok = v0 + j * 256 + (int)threadIdx.x < V;
    const uint32_t key = kv[j];
    if (PASS == 0) {
      if (ok) atomicAdd(&h[key >> 21], 1u);
    } else {
      if (ok && (key >> 21) == prefix) atomicAdd(&h[(key >> 10) & 2047u], 1u);
    }
  }
  __syncthreads();
  uint32_t* hh = hist + ((size_t)b * 3 + PASS) * 2048;
  for (int i = threadIdx.x; i < NBINS; i += 256)
    if (h[i]) atomicAdd(&hh[i], h[i]);
}

// The selection after the second radix pass, in two launches instead of a
// third pass, a count and a compaction over all the keys.  Every id whose
// key's top 22 bits are at least the selected prefix is a candidate: K plus
// the few other ids of that prefix (the first pass's 11-bit bins of float
// keys are a quarter octave wide and can hold much of the vocabulary; 22-bit
// ones hold a handful).  pool_collect_kernel compacts the candidates of
// every kPoolChunk ids, as (key, id) pairs in id order, into those ids' own
// stretch of cand (no counter shared between workgroups: same-line atomics
// from many workgroups serialise) and adds the candidates of the selected
// prefix to the last radix histogram; pool_select_kernel, one workgroup per
// request, takes the threshold from that histogram and writes the pool in id
// order: every key above the threshold and the lowest ids of those equal to
// it.
template <int F>
__global__ __launch_bounds__(256) void pool_collect_kernel(const uint32_t* __restrict__ keys, int V,
                                                           uint32_t* __restrict__ state,
                                                           uint32_t* __restrict__ hist,
                                                           uint2* __restrict__ cand,
                                                           uint32_t* __restrict__ cand_n, int nch) {
  constexpr int NL = F * kPoolChunk / 256;
  __shared__ int lds[4];
  __shared__ uint32_t res[2];
  __shared__ int wcnt[NL][4];  // candidates per (load, wave)
  const int b = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int v0 = blockIdx.x * F * kPoolChunk;
  uint32_t kv[NL];  // issued before the selection, which they do not depend on
#pragma unroll
  for (int j = 0; j < NL; ++j) kv[j] = keys[(size_t)b * V + min(v0 + j * 256 + (int)threadIdx.x, V - 1)];
  uint32_t* sb = state + 8 * b + 2;
  const uint2 ns = select_bin<1>(hist + ((size_t)b * 3 + 1) * 2048, sb[0], sb[1], lds, res);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    sb[2] = ns.x;
    sb[3] = ns.y;
  }
  uint64_t mk[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const bool ok = v0 + j * 256 + (int)threadIdx.x < V;
    mk[j] = __ballot(ok && (kv[j] >> 10) >= ns.x);
    if (lane == 0) wcnt[j][w] = __popcll(mk[j]);
    // the ids of the prefix itself go to the last histogram: few, but when
    // scores tie many, so a wave adds its lanes of the leader's bin at once
    const bool pe = ok && (kv[j] >> 10) == ns.x;
    const uint64_t pm = __ballot(pe);
    if (pm) {
      const int leader = __ffsll((unsigned long long)pm) - 1;
      const uint32_t lb = __shfl(kv[j] & 1023u, leader, 64);
      const uint64_t same = __ballot(pe && (kv[j] & 1023u) == lb);
      uint32_t* const h2 = hist + ((size_t)b * 3 + 2) * 2048;
      if (lane == leader) atomicAdd(&h2[lb], (uint32_t)__popcll(same));
      if (pe && (kv[j] & 1023u) != lb) atomicAdd(&h2[kv[j] & 1023u], 1u);
    }
  }
  __syncthreads();
  // each kPoolChunk ids (four loads) keep their candidates in their own
  // stretch, in id order, which is (load j, wave, lane)
  const uint64_t lt = (1ull << lane) - 1ull;
  int acc = 0;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    constexpr int per = kPoolChunk / 256;
    if (j % per == 0) acc = 0;
    int before = acc;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      before += x < w ? wcnt[j][x] : 0;
      acc += wcnt[j][x];
    }
    const int sub = v0 + (j / per) * kPoolChunk;
    if ((mk[j] >> lane) & 1ull)
      cand[(size_t)b * V + sub + before + __popcll(mk[j] & lt)] =
          make_uint2(kv[j], (uint32_t)(v0 + j * 256 + (int)threadIdx.x));
    if (j % per == per - 1 && threadIdx.x == 0 && sub < V)
      cand_n[(size_t)b * nch + sub / kPoolChunk] = (uint32_t)acc;
  }
}

// block-wide exclusive scans of two values at once (256 threads)
__device__ __forceinline__ int2 block_excl_scan2_256(int a, int c, int* lds8) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = a, y = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int px = __shfl_up(x, d, 64), py = __shfl_up(y, d, 64);
    if (lane >= d) {
      x += px;
      y += py;
    }
  }
  if (lane == 63) {
    lds8[w] = x;
    lds8[4 + w] = y;
  }
  __syncthreads();
  int ox = 0, oy = 0;
  for (int i = 0; i < w; ++i) {
    ox += lds8[i];
    oy += lds8[4 + i];
  }
  __syncthreads();
  return make_int2(ox + x - a, oy + y - c);
}

constexpr int kSelectPre = 24;  // candidates per thread loaded before the selection

// 256 threads (select_bin's scans) per request.  Thread t owns a run of
// consecutive chunks of kPoolChunk ids, so its candidates, in order, are a
// run of the ids in order.  Every load of the common case (the first
// chunk's count and up to kSelectPre candidates, read at clamped places
// inside that chunk's stretch before their number is known) is issued
// before the selection; more candidates (many equal scores) and further
// chunks (vocabularies above 256 chunks) are read in the walks.  With gt and
// eq the keys above and equal to the threshold before a thread's run, its
// first selected id goes to place gt + min(eq, need).
__global__ __launch_bounds__(256) void pool_select_kernel(
    int K, int nch, const uint32_t* __restrict__ state, const uint32_t* __restrict__ hist,
    const uint2* __restrict__ cand, const uint32_t* __restrict__ cand_n, int V,
    int32_t* __restrict__ pool_ids, uint32_t* __restrict__ umask, int ug) {
  __shared__ int lds[8];
  __shared__ uint32_t res[2];
  const int b = blockIdx.x;
  const uint2* const cb = cand + (size_t)b * V;
  const uint32_t* const nb = cand_n + (size_t)b * nch;
  const int cpt = (nch + 255) / 256;
  const int c0 = min((int)threadIdx.x * cpt, nch), c1 = min(c0 + cpt, nch);
  const bool any = c0 < c1;
  // the histogram first: the selection waits for it, not for the candidates
  SelectBins<2> bins;
  bins.load(hist + ((size_t)b * 3 + 2) * 2048);
  const uint2* const src0 = cb + (size_t)min(c0, nch - 1) * kPoolChunk;
  const int last = min(kPoolChunk, V - min(c0, nch - 1) * kPoolChunk) - 1;  // in the stretch
  uint2 e[kSelectPre];
#pragma unroll
  for (int j = 0; j < kSelectPre; ++j) e[j] = src0[min(j, last)];
  const int n0 = any ? (int)nb[c0] : 0;
  const uint2 s2 = select_bin<2>(bins, state[8 * b + 4], state[8 * b + 5], lds, res);
  const uint32_t T = s2.x;         // the K-th largest key
  const int need = (int)s2.y;      // keys equal to T to take, lowest ids first
  // f on candidates j0 .. n - 1 of a chunk's stretch, 4 loads at a time (more code made
  // the common path, which never gets here, slower)
  auto tail = [&](const uint2* src, int j0, int n, auto&& f) {
    for (int j = j0; j < n; j += 4) {
      uint2 t[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = src[min(j + i, n - 1)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j + i < n) f(t[i]);
    }
  };
  // f on this thread's candidates in id order
  auto walk = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < kSelectPre; ++j)
      if (j < n0) f(e[j]);
    tail(src0, kSelectPre, n0, f);
    for (int c = c0 + 1; c < c1; ++c) tail(cb + (size_t)c * kPoolChunk, 0, (int)nb[c], f);
  };
  int my_gt = 0, my_eq = 0;
  walk([&](uint2 x) {
    my_gt += x.x > T;
    my_eq += x.x == T;
  });
  const int2 before = block_excl_scan2_256(my_gt, my_eq, lds);
  int pos = before.x + min(before.y, need), eq = before.y;
  int32_t* const out = pool_ids + (size_t)b * K;
  walk([&](uint2 x) {
    const bool sel = x.x > T || (x.x == T && eq < need);
    eq += x.x == T;
    if (sel) {
      if (pos < K) {
        out[pos] = (int32_t)x.y;
        if (umask) atomicOr(&umask[(size_t)(b / ug) * V + x.y], 1u << (b % ug));
      }
      ++pos;
    }
  });
}

// ------------------------------------------------------ pool row unions
// For each group of ug requests, the union of their pools in id
// order: one row per id that some request of the group selected, with the
// bits of the requests that did.  A row's members take consecutive slots of
// the group's member arrays (row order, then request order), so the base
// value of (row, request) sits at the row's first slot plus the number of
// lower member bits.

// base logits of steps 1..14 at the pool ids, [14, B, K]: one thread per
// entry (ids ascend along a request's pool, so neighbouring threads read
// nearby ids of the same base row)
__global__ __launch_bounds__(256) void pool_gather_kernel(const int32_t* __restrict__ pool_ids,
                                                          const float* __restrict__ base, int V,
                                                          int B, int K,
                                                          float* __restrict__ pool_base) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n = (size_t)B * K;
  if (idx >= n * DOMINO_S) return;
  const int t = (int)(idx / n);
  const size_t bj = idx - (size_t)t * n;  // b * K + j
  const int b = (int)(bj / K);
  pool_base[idx] = base[((size_t)(t + 1) * B + b) * V + pool_ids[bj]];
}

// union rows and members per (group, id chunk)
__global__ __launch_bounds__(256) void union_count_kernel(const uint32_t* __restrict__ umask,
                                                          int V, uint32_t* __restrict__ ucounts,
                                                          int nch) {
  __shared__ int lds[4];
  const int g = blockIdx.y, v0 = blockIdx.x * kPoolChunk;
  int rows = 0, mem = 0;
#pragma unroll
  for (int j = 0; j < kPoolChunk / 256; ++j) {
    const int v = v0 + j * 256 + threadIdx.x;
    const uint32_t mv = umask[(size_t)g * V + min(v, V - 1)];  // clamped: issued unconditionally
    const uint32_t m = v < V ? mv : 0u;
    rows += m != 0u;
    mem += __popc(m);
  }
  rows = block_sum_256(rows, lds);
  mem = block_sum_256(mem, lds);
  if (threadIdx.x == 0) {
    ucounts[((size_t)g * nch + blockIdx.x) * 2] = (uint32_t)rows;
    ucounts[((size_t)g * nch + blockIdx.x) * 2 + 1] = (uint32_t)mem;
  }
}

// union rows in id order: records and the id -> row map; clears the masks
__global__ __launch_bounds__(256) void union_compact_kernel(
    uint32_t* __restrict__ umask, const bf16_t* __restrict__ b2, int V,
    const uint32_t* __restrict__ ucounts, int nch, uint4* __restrict__ urec, int32_t* __restrict__ uidx, int32_t* __restrict__ un, int umax) {
  __shared__ int lds[4];
  const int g = blockIdx.y, chunk = blockIdx.x;
  int rows_b = 0, mem_b = 0;
  for (int c = threadIdx.x; c < chunk; c += 256) {
    rows_b += (int)ucounts[((size_t)g * nch + c) * 2];
    mem_b += (int)ucounts[((size_t)g * nch + c) * 2 + 1];
  }
  rows_b = block_sum_256(rows_b, lds);
  mem_b = block_sum_256(mem_b, lds);
  // four consecutive ids per thread keep the scan order equal to id order
  const int v0 = chunk * kPoolChunk + threadIdx.x * 4;
  uint32_t m[4];
  int my_rows = 0, my_mem = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = v0 + j;
    m[j] = v < V ? umask[(size_t)g * V + v] : 0u;
    my_rows += m[j] != 0u;
    my_mem += __popc(m[j]);
  }
  int tot_rows = 0;
  int rpos = rows_b + block_excl_scan_256(my_rows, lds, &tot_rows);
  int mpos = mem_b + block_excl_scan_256(my_mem, lds, nullptr);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (m[j] == 0u) continue;
    const int v = v0 + j;
    if (rpos < umax) {  // always: a group's union has at most ug * K <= umax rows
      urec[(size_t)g * umax + rpos] =
          make_uint4((uint32_t)v, __float_as_uint(bf16_to_f32(b2[v])), (uint32_t)mpos, m[j]);
      uidx[(size_t)g * V + v] = rpos;
    }
    umask[(size_t)g * V + v] = 0u;
    ++rpos;
    mpos += __popc(m[j]);
  }
  if (chunk == nch - 1 && threadIdx.x == 0) un[g] = rows_b + tot_rows;
}

// base logits of steps 1..14 at every member, in the group's slot order,
// read straight from the base logits (all 14 loads issued with the row
// index, before the record that depends on it)
__global__ __launch_bounds__(256) void union_members_kernel(
    const int32_t* __restrict__ pool_ids, const float* __restrict__ base, int B, int K, int V,
    const int32_t* __restrict__ uidx, const uint4* __restrict__ urec, int umax,
    float* __restrict__ mb, int mstride, int ug, int ugmax) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= B * K) return;
  const int b = idx / K;
  const int g = b / ug, bl = b % ug;
  const int v = pool_ids[idx];
  // the row index and the 14 base values in one round trip, then the record;
  // the values are used once, so their lines are not kept in L2 (45 -> 40 us
  // at 8B, 64 requests, K = 2048)
  const int ui = uidx[(size_t)g * V + v];
  float vals[DOMINO_S];
#pragma unroll
  for (int t = 0; t < DOMINO_S; ++t)
    vals[t] = __builtin_nontemporal_load(&base[((size_t)(t + 1) * B + b) * V + v]);
  __builtin_amdgcn_sched_barrier(0);
  const uint4 rc = urec[(size_t)g * umax + ui];
  const uint32_t slot = rc.z + __popc(rc.w & ((1u << bl) - 1u));
#pragma unroll
  for (int t = 0; t < DOMINO_S; ++t) mb[((size_t)t * ugmax + g) * mstride + slot] = vals[t];
}

// The whole-line pool gather (correct_pool_lines_kernel) serves bf16 models
// up to this many requests, when the pool is not read as group unions.
// Measured at the 8B shapes, K = 2048 (us per correction, whole lines /
// fragments): B = 1 5.6 / 6.1, 2 8.3 / 8.1, 4 11.8 / 13.6, 8 16.8 / 21.0,
// 12 21.2 / 26.0, 16 43.9 / 33.3.  It reads each candidate's base logit from
// the step's base row itself, so the build skips the base-value gather.
constexpr int kPoolLinesMaxBatch = 12;
static bool pool_lines(const Shape& s, int B) {
  return s.bf16 && B <= kPoolLinesMaxBatch && s.r <= 512 * 3;
}

template <int F>
static void pool_select_passes(const Shape& s, const Workspace& ws, int B, int K, bool keys_ready,
                               bool hist_ready, bool uni, hipStream_t st) {
  const int nch = (s.V + F * kPoolChunk - 1) / (F * kPoolChunk);
  const dim3 grid(nch, B), blk(256);
  if (hist_ready) {
    // the LM-head counted the keys itself
  } else if (keys_ready) {
    DLAUNCH((pool_hist_kernel<0, F>), grid, blk, 0, st, ws.keys, s.V, ws.state, ws.hist, K);
  } else {
    DLAUNCH((pool_score_hist_kernel<F>), grid, blk, 0, st, ws.base, s.V, B, ws.keys, ws.hist);
  }
  DLAUNCH((pool_hist_kernel<1, F>), grid, blk, 0, st, ws.keys, s.V, ws.state, ws.hist, K);
  const int nsub = (s.V + kPoolChunk - 1) / kPoolChunk;
  DLAUNCH((pool_collect_kernel<F>), grid, blk, 0, st, ws.keys, s.V, ws.state, ws.hist, ws.cand,
          ws.cand_n, nsub);
  DLAUNCH(pool_select_kernel, dim3(B), blk, 0, st, K, nsub, ws.state, ws.hist, ws.cand,
          ws.cand_n, s.V, ws.pool_ids, uni ? ws.umask : nullptr, ws.ugroup);
}

void launch_pool_build(const Shape& s, const Workspace& ws, const void* fc2_b, int B, int K,
                       bool keys_ready, bool hist_ready, hipStream_t st) {
  const int nch = (s.V + kPoolChunk - 1) / kPoolChunk;  // union kernels: kPoolChunk ids per chunk
  const dim3 blk(256);
  const bool uni = pool_union(s, ws, B, K);
  if (B >= kPoolChunk4MinBatch)
    pool_select_passes<4>(s, ws, B, K, keys_ready, hist_ready, uni, st);
  else if (B >= kPoolChunk2MinBatch)
    pool_select_passes<2>(s, ws, B, K, keys_ready, hist_ready, uni, st);
  else
    pool_select_passes<1>(s, ws, B, K, keys_ready, hist_ready, uni, st);
  if (uni) {
    const dim3 ug(nch, (B + ws.ugroup - 1) / ws.ugroup);
    DLAUNCH(union_count_kernel, ug, blk, 0, st, ws.umask, s.V, ws.ucounts, nch);
    DLAUNCH(union_compact_kernel, ug, blk, 0, st, ws.umask, (const bf16_t*)fc2_b, s.V,
            ws.ucounts, nch, ws.urec, ws.uidx, ws.un, ws.umax);
    DLAUNCH(union_members_kernel, dim3((B * K + 255) / 256), blk, 0, st, ws.pool_ids, ws.base, B,
            K, s.V, ws.uidx, ws.urec, ws.umax, ws.mb, ws.mstride, ws.ugroup, ws.ugmax);
  } else if (!pool_lines(s, B)) {  // the whole-line gather reads base rows itself
    const size_t n = (size_t)B * K * DOMINO_S;
    DLAUNCH(pool_gather_kernel, dim3((unsigned)((n + 255) / 256)), blk, 0, st, ws.pool_ids,
            ws.base, s.V, B, K, ws.pool_base);
  }
}

// ------------------------------------------------- correction, full vocabulary
// y[b,c] = base[k,b,c] + (fc2[c]·u_b + b2[c]) for every vocabulary id c,
// then the argmax per request.  Each wave streams RT tiles of 16 fc2 rows
// once and multiplies them with all B requests' u (NB column blocks of 16).
template <bool BF>
struct CorrArgs {
  const W_t<BF>* F2;
  const W_t<BF>* b2;
  const float* base_k;   // base row k: [B, V]
  const float* u;
  const uint16_t* u_hi;
  const uint16_t* u_lo;
  uint64_t* slot_k;      // [B]
  int B, V, r;
};

template <bool BF>
__device__ __forceinline__ void load_u_frag(const CorrArgs<BF>& a, int b, int k, bool ok,
                                            HFrag<BF>& f) {
  if constexpr (BF) {
    const size_t off = (size_t)b * a.r + k;
    f.hi = ok ? load_frag_bf16(a.u_hi + off) : zero_frag();
    f.lo = ok ? load_frag_bf16(a.u_lo + off) : zero_frag();
  } else {
    f.f = ok ? load8_f32(a.u + (size_t)b * a.r + k) : zero8();
  }
}

template <bool BF, int NB, int RT>
__global__ __launch_bounds__(256) void correct_full_kernel(CorrArgs<BF> a) {
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;
  const int tile0 = (blockIdx.x * 4 + wave) * RT;
  const int V = a.V, r = a.r;
  const bool active = tile0 * 16 < V;

  uint64_t best[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) best[cb] = 0;

  if (active) {
    const W_t<BF>* pa[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int c = (tile0 + t) * 16 + row;
      pa[t] = a.F2 + (size_t)min(c, V - 1) * r + q * 8;
    }
    v4f acc[RT][NB];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) acc[t][cb] = zero4();
    for (int k = 0; k < r; k += 32) {
      WFrag<BF> A[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) A[t].load(pa[t] + k);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int b = cb * 16 + row;
        HFrag<BF> uf;
        load_u_frag<BF>(a, b, k + q * 8, b < a.B, uf);
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t][cb] = mma(A[t], uf, acc[t][cb]);
      }
    }
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int b = cb * 16 + row;
      if (b >= a.B) continue;
      const float* brow = a.base_k + (size_t)b * V;
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = (tile0 + t) * 16 + 4 * q + i;
          if (c < V) {
            const float y = brow[c] + (acc[t][cb][i] + load_w<BF>(a.b2 + c));
            best[cb] = umax64(best[cb], pack_key(y, (uint32_t)c));
          }
        }
    }
  }
  // lanes row, row+16, row+32, row+48 hold the same column
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    best[cb] = umax64(best[cb], shfl_xor_u64(best[cb], 16));
    best[cb] = umax64(best[cb], shfl_xor_u64(best[cb], 32));
  }
  __shared__ uint64_t wb[4][NB][16];
  if (q == 0)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) wb[wave][cb][row] = best[cb];
  __syncthreads();
  if (threadIdx.x < NB * 16) {
    const int cb = threadIdx.x >> 4, n = threadIdx.x & 15;
    const int b = cb * 16 + n;
    if (b < a.B) {
      const uint64_t m = umax64(umax64(wb[0][cb][n], wb[1][cb][n]), umax64(wb[2][cb][n], wb[3][cb][n]));
      publish_slot(a.slot_k, b, m);
    }
  }
}

constexpr int kCorrRT = 4;
// consecutive correction steps stream fc2 in opposite k order
constexpr bool kReverseOddSteps = true;

template <bool BF, int NB>
static void correct_full_launch(const CorrArgs<BF>& a, hipStream_t st) {
  const int tiles = (a.V + 15) / 16;
  const int units = (tiles + kCorrRT - 1) / kCorrRT;
  DLAUNCH((correct_full_kernel<BF, NB, kCorrRT>), dim3((units + 3) / 4), dim3(256), 0,
                     st, a);
}
template <bool BF>
static void correct_full_dispatch(const CorrArgs<BF>& a, hipStream_t st) {
  switch ((a.B + 15) / 16) {
    case 1: correct_full_launch<BF, 1>(a, st); break;
    case 2: correct_full_launch<BF, 2>(a, st); break;
    case 3: correct_full_launch<BF, 3>(a, st); break;
    default: correct_full_launch<BF, 4>(a, st); break;
  }
}

void launch_correct_full(const Shape& s, const DeviceWeights& w, const Workspace& ws, int k, int B,
                         hipStream_t st) {
  const float* base_k = ws.base + (size_t)k * B * s.V;
  uint64_t* slot_k = ws.slots + (size_t)k * B * kSlotSpan;
  if (s.bf16 && rowstream_supported(s.r, B)) {
    StreamArgs a{(const uint16_t*)w.fc2, s.V, s.r, ws.u_hi, ws.u_lo, B, 0, 0, nullptr,
                 (const uint16_t*)w.fc2_b, base_k, slot_k, kReverseOddSteps ? (k & 1) : 0};
    a.Wpk = B >= kPackedStreamMinBatch ? ws.fc2p : nullptr;
    launch_rowstream_argmax(a, st);
  } else if (s.bf16) {
    CorrArgs<true> a{(const bf16_t*)w.fc2, (const bf16_t*)w.fc2_b, base_k, ws.u, ws.u_hi, ws.u_lo,
                     slot_k, B, s.V, s.r};
    correct_full_dispatch<true>(a, st);
  } else {
    CorrArgs<false> a{(const float*)w.fc2, (const float*)w.fc2_b, base_k, ws.u, ws.u_hi, ws.u_lo,
                      slot_k, B, s.V, s.r};
    correct_full_dispatch<false>(a, st);
  }
}

// ------------------------------------------------------ correction, pool
// Per request, 16 gathered fc2 rows form the A tile; u_b sits in column 0
// (bf16 models: hi in column 0, lo in column 1) of the B tile.
template <bool BF>
struct PoolArgs {
  const W_t<BF>* F2;
  const W_t<BF>* b2;
  const float* pool_base_k;  // [B, K] base logits of step k at the pool ids
  const int32_t* pool_ids;   // [B, K]
  const float* u;
  const uint16_t* u_hi;
  const uint16_t* u_lo;
  uint64_t* slot_k;
  int B, K, r, V, units_per_req;
  const float* base_k;       // [B, V] base row of step k (whole-line gather)
};

template <bool BF, int RT>
__global__ __launch_bounds__(256) void correct_pool_kernel(PoolArgs<BF> a) {
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;
  const int unit = blockIdx.x * 4 + wave;
  const int b = unit / a.units_per_req;
  if (b >= a.B) return;  // no workgroup barrier below
  const int tile0 = (unit % a.units_per_req) * RT;
  const int K = a.K, r = a.r;
  const int32_t* ids = a.pool_ids + (size_t)b * K;

  const W_t<BF>* pa[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int i = (tile0 + t) * 16 + row;
    const int id = min(max(ids[min(i, K - 1)], 0), a.V - 1);  // ids are in range by construction
    pa[t] = a.F2 + (size_t)id * r + q * 8;
  }
  v4f acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = zero4();
  for (int k = 0; k < r; k += 32) {
    WFrag<BF> A[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) A[t].load(pa[t] + k);
    HFrag<BF> uf;
    if constexpr (BF) {
      const size_t off = (size_t)b * r + k + q * 8;
      uf.hi = row == 0 ? load_frag_bf16(a.u_hi + off) : (row == 1 ? load_frag_bf16(a.u_lo + off) : zero_frag());
      uf.lo = zero_frag();
      // one product per tile: the lo half rides in column 1
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t] = mfma_bf16(A[t].f, uf.hi, acc[t]);
    } else {
      uf.f = row == 0 ? load8_f32(a.u + (size_t)b * r + k + q * 8) : zero8();
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t] = mma(A[t], uf, acc[t]);
    }
  }
  uint64_t best = 0;
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float dot = acc[t][i];
      if (BF) dot += __shfl_down(acc[t][i], 1, 64);  // column 1 (lo) of the same row
      const int idx = (tile0 + t) * 16 + 4 * q + i;
      if (row == 0 && idx < K) {
        const int id = min(max(ids[idx], 0), a.V - 1);
        const float y = a.pool_base_k[(size_t)b * K + idx] + (dot + load_w<BF>(a.b2 + id));
        best = umax64(best, pack_key(y, (uint32_t)id));
      }
    }
  best = wave_max_u64(best);
  if (lane == 0) publish_slot(a.slot_k, b, best);
}

// bf16 pool correction with the projector width split over the four waves
// of a workgroup: one workgroup per 16 gathered candidates of one request,
// every wave with all of its fc2 loads in flight at once (latency bound at
// small batch, so parallelism matters more than reuse).
template <int CPW>  // 32-wide k chunks per wave
__global__ __launch_bounds__(256) void correct_pool_split_kernel(PoolArgs<true> a) {
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;
  const int tiles = (a.K + 15) / 16;
  const int b = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int K = a.K, r = a.r;
  const int32_t* ids = a.pool_ids + (size_t)b * K;
  const int i = tile * 16 + row;
  const int id = min(max(ids[min(i, K - 1)], 0), a.V - 1);
  const bf16_t* pa = a.F2 + (size_t)id * r + q * 8;
  const size_t uoff = (size_t)b * r + q * 8;
  const int nch = r / 32;
  v8s A[CPW], U[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int k = min(wave + 4 * c, nch - 1) * 32;  // chunks past the width are masked below
    A[c] = load_frag_bf16(pa + k);
    U[c] = row == 0 ? load_frag_bf16(a.u_hi + uoff + k)
                    : (row == 1 ? load_frag_bf16(a.u_lo + uoff + k) : zero_frag());
  }
  v4f acc = zero4();
#pragma unroll
  for (int c = 0; c < CPW; ++c)
    if (wave + 4 * c < nch) acc = mfma_bf16(A[c], U[c], acc);
  __shared__ float red[4][4][64];
#pragma unroll
  for (int e = 0; e < 4; ++e) red[wave][e][lane] = acc[e];
  __syncthreads();
  if (wave != 0) return;  // no barrier below
  uint64_t best = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float part = ((red[0][e][lane] + red[1][e][lane]) + red[2][e][lane]) + red[3][e][lane];
    const float dot = part + __shfl_down(part, 1, 64);  // hi (column 0) + lo (column 1)
    const int idx = tile * 16 + 4 * q + e;
    if (row == 0 && idx < K) {
      const int cid = min(max(ids[idx], 0), a.V - 1);
      const float y = a.pool_base_k[(size_t)b * K + idx] + (dot + bf16_to_f32(a.b2[cid]));
      best = umax64(best, pack_key(y, (uint32_t)cid));
    }
  }
  best = wave_max_u64(best);
  if (lane == 0) publish_slot(a.slot_k, b, best);
}

// bf16 pool correction with whole-line loads, for small batches: one wave
// per 16 candidates of one request.  Lane l reads elements 512 p + 8 l .. +7
// of every candidate's fc2 row (one 16-byte load per 512-wide piece p), so a
// load instruction covers 1 KB of one row, eight whole 128-byte lines, where
// a matrix-core fragment would touch sixteen rows at 64 bytes each.  The dots
// are fp32 FMAs of the bf16 weights against u in fp32 (the work is tiny:
// 2 r flops per candidate); a transposed butterfly finishes all 16 dots of a
// wave with 17 shuffles, leaving candidate (l >> 2) & 15 in lanes 4i..4i+3.
// The epilogue operands (the candidate's id, then its base logit, read from
// the step's base row, and its bias) are loaded before the weights arrive.
template <int NP>
__global__ __launch_bounds__(256) void correct_pool_lines_kernel(PoolArgs<true> a) {
  const int lane = threadIdx.x & 63;
  const int K = a.K, r = a.r;
  const int tiles = (K + 15) / 16;
  const int unit = blockIdx.x * 4 + wave_index();
  const int b = unit / tiles;
  if (b >= a.B) return;  // no barrier in this kernel
  const int tile = unit - b * tiles;
  const int32_t* ids = a.pool_ids + (size_t)b * K;
  // the id of candidate lane % 16 (row addresses), and of this lane's result row
  const int myid = min(max(ids[min(tile * 16 + (lane & 15), K - 1)], 0), a.V - 1);
  const int rr = (lane >> 2) & 15, ridx = tile * 16 + rr;
  const int rid = min(max(ids[min(ridx, K - 1)], 0), a.V - 1);
  const float rbase = a.base_k[(size_t)b * a.V + rid];
  const float rbias = bf16_to_f32(a.b2[rid]);
  float uf[NP][8];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int k = 512 * p + 8 * lane;
    const bool ok = k < r;
    const F8 v = load8_f32(a.u + (size_t)b * r + (ok ? k : 0));
#pragma unroll
    for (int e = 0; e < 8; ++e) uf[p][e] = ok ? v.v[e] : 0.f;
  }
  uint4 w[16][NP];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bf16_t* row = a.F2 + (size_t)__shfl(myid, i, 64) * r;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int k = 512 * p + 8 * lane;
      w[i][p] = *reinterpret_cast<const uint4*>(row + (k < r ? k : 0));  // masked by uf = 0
    }
  }
  float d[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t x[4] = {w[i][p].x, w[i][p].y, w[i][p].z, w[i][p].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(__uint_as_float(x[e] << 16), uf[p][2 * e], acc);
        acc = fmaf(__uint_as_float(x[e] & 0xFFFF0000u), uf[p][2 * e + 1], acc);
      }
    }
    d[i] = acc;
  }
  // transposed butterfly: after the step over lane bit m, a lane keeps the
  // half of its values whose row index has that bit equal to its own
  const bool h5 = lane & 32, h4 = lane & 16, h3 = lane & 8, h2 = lane & 4;
  float e8[8], e4[4], e2[2];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    e8[j] = (h5 ? d[8 + j] : d[j]) + __shfl_xor(h5 ? d[j] : d[8 + j], 32, 64);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    e4[j] = (h4 ? e8[4 + j] : e8[j]) + __shfl_xor(h4 ? e8[j] : e8[4 + j], 16, 64);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    e2[j] = (h3 ? e4[2 + j] : e4[j]) + __shfl_xor(h3 ? e4[j] : e4[2 + j], 8, 64);
  float dot = (h2 ? e2[1] : e2[0]) + __shfl_xor(h2 ? e2[0] : e2[1], 4, 64);
  dot += __shfl_xor(dot, 2, 64);
  dot += __shfl_xor(dot, 1, 64);
  const float y = rbase + (dot + rbias);
  uint64_t best = (ridx < K) ? pack_key(y, (uint32_t)rid) : 0ull;
  best = wave_max_u64(best);
  if (lane == 0) publish_slot(a.slot_k, b, best);
}

constexpr int kPoolRT = 2;
constexpr int kPoolSplitMaxBatch = 16;


// Above the small-batch split kernel, bf16 pools can be corrected by
// streaming each request group's union of pool rows once through the
// persistent kernel (every pool row is read once per group instead of once
// per request holding it; the group's products come from one pass over the
// row).  Building the unions costs ~20 us per block, so the automatic choice
// takes them once the per-request gather would read enough per step:
// kUnionMinGatherBytes above 16 requests (measured at 8B shapes, B = 64: the
// gather wins at K <= 512, the unions from K = 1024 on), half of it for the
// latency-bound small-batch gather (B = 16, K = 2048: unions 1.13 against
// 1.27 ms per block; B = 8: even).
constexpr long long kUnionMinGatherBytes = 96ll << 20;
static int union_bound(const Shape& s, const Workspace& ws, int K) {
  return (int)std::min<long long>(s.V, (long long)ws.ugroup * K);
}

bool pool_union(const Shape& s, const Workspace& ws, int B, int K) {
  if (!(s.bf16 && ws.umask != nullptr && ws.ugroup > 0 && B <= ws.ugroup * ws.ugmax &&
        rowstream_union_supported(s.r, B, union_bound(s, ws, K), ws.ugroup)) ||
      ws.pool_strategy == 1)
    return false;
  const long long gather = (long long)B * K * s.r * 2;
  return ws.pool_strategy == 2 ||
         gather >= (B > kPoolSplitMaxBatch ? kUnionMinGatherBytes : kUnionMinGatherBytes / 2);
}

void launch_correct_pool(const Shape& s, const DeviceWeights& w, const Workspace& ws, int k, int B,
                         int K, hipStream_t st) {
  const int tiles = (K + 15) / 16;
  const int upr = (tiles + kPoolRT - 1) / kPoolRT;  // units per request (fp32 / wide kernels)
  const int units = upr * B;
  const dim3 grid((units + 3) / 4);
  const float* pb = ws.pool_base + (size_t)(k - 1) * B * K;
  uint64_t* slot_k = ws.slots + (size_t)k * B * kSlotSpan;
  if (pool_union(s, ws, B, K)) {
    StreamArgs a{(const uint16_t*)w.fc2, 0, s.r, ws.u_hi, ws.u_lo, B, 0, 0, nullptr,
                 nullptr, nullptr, slot_k, kReverseOddSteps ? (k & 1) : 0};
    a.urec = ws.urec;
    a.un = ws.un;
    a.mb_k = ws.mb + (size_t)(k - 1) * ws.ugmax * ws.mstride;
    a.ustride = ws.umax;
    a.mstride = ws.mstride;
    launch_rowstream_union(a, union_bound(s, ws, K), ws.ugroup, st);
    return;
  }
  // small batches are latency bound: spread each request's pool over many workgroups
  if (pool_lines(s, B)) {
    PoolArgs<true> a{(const bf16_t*)w.fc2, (const bf16_t*)w.fc2_b, pb, ws.pool_ids, ws.u, ws.u_hi,
                     ws.u_lo, slot_k, B, K, s.r, s.V, upr};
    a.base_k = ws.base + (size_t)k * B * s.V;
    const dim3 g4((unsigned)((B * tiles + 3) / 4));
    switch ((s.r + 511) / 512) {
      case 1: DLAUNCH((correct_pool_lines_kernel<1>), g4, dim3(256), 0, st, a); break;
      case 2: DLAUNCH((correct_pool_lines_kernel<2>), g4, dim3(256), 0, st, a); break;
      default: DLAUNCH((correct_pool_lines_kernel<3>), g4, dim3(256), 0, st, a); break;
    }
  } else if (s.bf16 && B <= kPoolSplitMaxBatch && s.r % 32 == 0 && s.r <= 32 * 4 * 12) {
    PoolArgs<true> a{(const bf16_t*)w.fc2, (const bf16_t*)w.fc2_b, pb, ws.pool_ids, ws.u, ws.u_hi,
                     ws.u_lo, slot_k, B, K, s.r, s.V, upr};
    const dim3 g2((unsigned)(B * tiles));
    switch ((s.r / 32 + 3) / 4) {
      case 1: DLAUNCH((correct_pool_split_kernel<1>), g2, dim3(256), 0, st, a); break;
      case 2: DLAUNCH((correct_pool_split_kernel<2>), g2, dim3(256), 0, st, a); break;
      case 3: DLAUNCH((correct_pool_split_kernel<3>), g2, dim3(256), 0, st, a); break;
      case 4: DLAUNCH((correct_pool_split_kernel<4>), g2, dim3(256), 0, st, a); break;
      case 5: DLAUNCH((correct_pool_split_kernel<5>), g2, dim3(256), 0, st, a); break;
      case 6: DLAUNCH((correct_pool_split_kernel<6>), g2, dim3(256), 0, st, a); break;
      case 7: DLAUNCH((correct_pool_split_kernel<7>), g2, dim3(256), 0, st, a); break;
      case 8: DLAUNCH((correct_pool_split_kernel<8>), g2, dim3(256), 0, st, a); break;
      case 9: DLAUNCH((correct_pool_split_kernel<9>), g2, dim3(256), 0, st, a); break;
      case 10: DLAUNCH((correct_pool_split_kernel<10>), g2, dim3(256), 0, st, a); break;
      case 11: DLAUNCH((correct_pool_split_kernel<11>), g2, dim3(256), 0, st, a); break;
      default: DLAUNCH((correct_pool_split_kernel<12>), g2, dim3(256), 0, st, a); break;
    }
  } else if (s.bf16) {
    PoolArgs<true> a{(const bf16_t*)w.fc2, (const bf16_t*)w.fc2_b, pb, ws.pool_ids, ws.u, ws.u_hi,
                     ws.u_lo, slot_k, B, K, s.r, s.V, upr};
    DLAUNCH((correct_pool_kernel<true, kPoolRT>), grid, dim3(256), 0, st, a);
  } else {
    PoolArgs<false> a{(const float*)w.fc2, (const float*)w.fc2_b, pb, ws.pool_ids, ws.u, ws.u_hi,
                      ws.u_lo, slot_k, B, K, s.r, s.V, upr};
    DLAUNCH((correct_pool_kernel<false, kPoolRT>), grid, dim3(256), 0, st, a);
  }
}

// ---------------------------------------------------------------- outputs
// One workgroup per request: lane k < P writes proposal k, then (after every
// lane has read them) the request's argmax words, bad flag and, after a pool
// run, radix histograms are cleared for the next run.
__global__ __launch_bounds__(64) void writeout_kernel(uint64_t* __restrict__ slots,
                                                      int32_t* __restrict__ bad,
                                                      uint32_t* __restrict__ hist, int B, int P,
                                                      int32_t* __restrict__ out_tokens,
                                                      float* __restrict__ out_top1) {
  const int b = blockIdx.x, k = threadIdx.x;
  const bool flagged = bad[b] != 0;
  if (k < P) {
    const uint64_t key = read_slot(slots, k * B + b);
    const bool invalid = flagged || key == 0;
    out_tokens[b * P + k] = invalid ? -1 : key_id(key);
    if (out_top1) out_top1[b * P + k] = invalid ? __builtin_nanf("") : key_value(key);
  }
  __syncthreads();  // every lane has read bad[b]
  for (int i = k; i < DOMINO_T * kSlotCopies; i += 64)
    slots[(size_t)((i / kSlotCopies) * B + b) * kSlotSpan + (i % kSlotCopies) * kSlotLine] = 0;
  if (k == 0) bad[b] = 0;
  if (hist)
    for (int i = k; i < 3 * 2048; i += 64) hist[(size_t)b * 3 * 2048 + i] = 0;
}

void launch_writeout(const Workspace& ws, int B, int P, bool pool, int32_t* out_tokens,
                     float* out_top1, hipStream_t st) {
  DLAUNCH(writeout_kernel, dim3(B), dim3(64), 0, st, ws.slots, ws.bad, pool ? ws.hist : nullptr,
          B, P, out_tokens, out_top1);
}
