// Base LM-head logits of a one-request block, full vocabulary:
//   base[t, 0, v] = sum_i hidden[0, t, i] * lm_head[v, i]      (fp32, t = 0..14)
// with, in the same pass, the request's pool score key orderable(max_t
// base[t, 0, v]) and the first proposal argmax_v base[0, 0, v].
// "Add correctness-first Domino support to DFlash V2" (sglang PR #31328),
// "Design": full-vocabulary base projection, first proposal = its argmax,
// the pool built from the block's base logits.
//
// At one request the LM-head is a stream of lm_head (1.25 GB at the 8B
// shapes) against 15 activation rows, so its speed is the speed of the
// weight stream.  On MI355X a load-only probe of a [151936, 4096] bf16
// matrix streamed 16 rows x 64 B per load instruction (the shape of an MFMA
// operand fragment) at 4.4 TB/s, but 4 rows x 256 B (whole 128-byte lines)
// at 5.8 TB/s (cached loads); direct global->LDS copies of the same lines
// reached only 1.8-3.7 TB/s.  This kernel therefore loads lm_head as whole
// lines into registers and turns them into fragments through LDS:
//  * The H/512 waves of a workgroup split K: wave w owns k in
//    [512 w, 512 w + 512) and keeps its 16 activation fragments (15 rows
//    plus a zero row, 64 VGPRs) in registers for the whole launch.
//  * A tile is 16 consecutive lm_head rows (128 KB at H = 4096).  With
//    non-temporal loads a probe of this kernel's load pattern streamed
//    consecutive rows as fast as rows ceil(V / 16) apart (182.8 / 182.7 us
//    at 8B), and consecutive rows make each workgroup's logits and keys one
//    contiguous range (whole-line stores: LM-head 192.7 -> 190.2 us, the
//    K = 2048 block 0.366 -> 0.363 ms).  A wave streams its K range of a
//    tile in two stages of 256 k, each eight loads of 4 rows x 256 B, the next stage in
//    flight while one is consumed.  (A deeper ring in registers made the
//    compiler wait for all but the newest stage at the loop head; with two
//    stages that wait is exactly the one needed.)  A stage goes through the
//    wave's own 8 KB of LDS (16-byte chunk c of row r at position
//    (c & 16) | ((c ^ r) & 15), so the row-wise writes and the 16-row
//    fragment reads hit distinct banks) and comes back as eight MFMA
//    operand fragments.  A wave only reads what it wrote, so the stream
//    needs no barrier.
//  * After its two stages each wave holds a 16 x 16 partial tile; the
//    partials meet in LDS (one barrier per tile), and the sums, the pool key
//    of each row and a running first-proposal maximum are kept; the sums and
//    keys stay in LDS (a global store inside the loop also made the compiler
//    over-wait) and are written after the last tile, consecutive threads
//    on consecutive ids.  The workgroup publishes its first-proposal word
//    once.
//  * A workgroup takes a contiguous range of t (ranges balanced to one tile),
//    one workgroup per CU.
//  * With a pool to build, the workgroup also counts its keys by their top
//    11 bits (the pool selection's first radix histogram) in LDS and adds
//    the nonzero bins to the histogram in memory, so the selection starts
//    at its second pass.
#include "common.h"
#include "launch.h"

namespace {

// A wave owns KS 32-wide k steps (32 KS of K) in KS / 4 stages of 128 k.
// load j of a stage (256 k at k offset kbase + 256 sub of tile t): rows
// 4 i .. 4 i + 3 (i = j % 4) of the j / 4-th 128-k block, lane l row
// 4 i + l / 16, chunk l % 16 of the block's 256 bytes.  W is deliberately not
// __restrict__ (with a restrict pointer to read-only data the optimizer
// moved loads next to their uses).  The loads are non-temporal: every line is
// read once, and lm_head lines kept in the L2s would only displace what the
// rest of the rollout reads (8B: 214 -> 193 us for this kernel, and the pool
// cell's block 0.410 -> 0.367 ms).
__device__ __forceinline__ uint4 one_ld(const bf16_t* W, int t, int sub, int j, int V, int H,
                                        int kbase, int row, int q) {
  const int i = j & 3, kb = j >> 2;
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
      W + kbase + 256 * sub + 128 * kb + 8 * row + (size_t)min(16 * t + 4 * i + q, V - 1) * H));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int WV, int KS>
__global__ __launch_bounds__(WV * 64) void lmhead_one_kernel(const bf16_t* W,
                                                             const bf16_t* __restrict__ X,
                                                             float* __restrict__ out,
                                                             uint32_t* __restrict__ keys,
                                                             uint32_t* __restrict__ hist0,
                                                             uint64_t* __restrict__ slot0, int V,
                                                             int H, int maxt) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;
  const int S = (V + 15) / 16;
  constexpr int SPT = KS / 8;  // stages per tile (256 k each)
  static_assert(SPT == 2, "two stages per tile: the ring is two stages deep");
  const int kbase = wave * (KS * 32);
  unsigned char* const buf = smem + wave * 8192;  // one 8 KB stage buffer
  float* const red = reinterpret_cast<float*>(smem + WV * 8192);  // [2][WV][256]
  // the workgroup's summed tiles [tile][column][row] and keys [tile][row]
  // (maxt tiles at most)
  float* const zout = red + 2 * WV * 256;
  uint32_t* const kout = reinterpret_cast<uint32_t*>(zout + maxt * 256);
  uint32_t* const hloc = kout + maxt * 16;  // [2048] keys by their top 11 bits
  for (int i = threadIdx.x; i < 2048; i += WV * 64) hloc[i] = 0;  // ordered by the tile barriers

  // this wave's activation fragments: column `row` (draft position; 15 is zero)
  v8s xf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const v8s v = load_frag_bf16(X + (size_t)min(row, DOMINO_T - 1) * H + kbase + 32 * s + 8 * q);
    xf[s] = row < DOMINO_T ? v : zero_frag();
  }

  // this workgroup's tiles: t in [t0, t0 + ntiles), ranges balanced to one tile
  const int t0 = (int)(((long long)blockIdx.x * S) / gridDim.x);
  const int ntiles = (int)(((long long)(blockIdx.x + 1) * S) / gridDim.x) - t0;

  // two stages in registers: stage g + 1 is loaded while stage g is consumed
  // (with a two-deep ring the compiler's wait at the loop head is exact)
  const int nst = ntiles * SPT;
  auto stage_tile = [&](int g) { return t0 + min(g, nst - 1) / SPT; };
  auto stage_sub = [&](int g) { return min(g, nst - 1) % SPT; };
  uint4 a0, a1, a2, a3, a4, a5, a6, a7, b0, b1, b2, b3, b4, b5, b6, b7;
#define ONE_LOAD8(G, X)                                                                          \
  {                                                                                              \
    const int tt_ = stage_tile(G), ss_ = stage_sub(G);                                           \
    X##0 = one_ld(W, tt_, ss_, 0, V, H, kbase, row, q);                                          \
    X##1 = one_ld(W, tt_, ss_, 1, V, H, kbase, row, q);                                          \
    X##2 = one_ld(W, tt_, ss_, 2, V, H, kbase, row, q);                                          \
    X##3 = one_ld(W, tt_, ss_, 3, V, H, kbase, row, q);                                          \
    X##4 = one_ld(W, tt_, ss_, 4, V, H, kbase, row, q);                                          \
    X##5 = one_ld(W, tt_, ss_, 5, V, H, kbase, row, q);                                          \
    X##6 = one_ld(W, tt_, ss_, 6, V, H, kbase, row, q);                                          \
    X##7 = one_ld(W, tt_, ss_, 7, V, H, kbase, row, q);                                          \
  }
#define ONE_PUT(J, X)                                                                            \
  {                                                                                              \
    const int r_ = 4 * ((J) & 3) + q, c_ = 16 * ((J) >> 2) + row;                                \
    *reinterpret_cast<uint4*>(buf + (r_ * 32 + ((c_ & 16) | ((c_ ^ r_) & 15))) * 16) = X;        \
  }
  ONE_LOAD8(0, a)

  uint64_t best0 = 0;  // first-proposal candidate (output threads of column 0)
  int par = 0;
  for (int n = 0; n < ntiles; ++n) {
    v4f acc = zero4();
    // stage SUB of the tile from registers CUR, with the next stage loaded
    // into NXT: into LDS (chunk c of row r at position (c & 16) | ((c ^ r) &
    // 15)), then eight fragments (row l % 16, chunk 4 s + l / 16) against the
    // wave's activations.  A wave's LDS operations run in order, so the next
    // stage's writes cannot overtake these reads.
#define ONE_STAGE(SUB, CUR, NXT)                                                                 \
    {                                                                                            \
      __builtin_amdgcn_sched_barrier(0);                                                         \
      ONE_LOAD8(n * SPT + (SUB) + 1, NXT)                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                         \
      ONE_PUT(0, CUR##0) ONE_PUT(1, CUR##1) ONE_PUT(2, CUR##2) ONE_PUT(3, CUR##3)                \
      ONE_PUT(4, CUR##4) ONE_PUT(5, CUR##5) ONE_PUT(6, CUR##6) ONE_PUT(7, CUR##7)                \
      _Pragma("unroll") for (int s = 0; s < 8; ++s) {                                            \
        const int c = 4 * s + q;                                                                 \
        const v8s a =                                                                            \
            *reinterpret_cast<const v8s*>(buf + (row * 32 + ((c & 16) | ((c ^ row) & 15))) * 16); \
        acc = mfma_bf16(a, xf[(SUB) * 8 + s], acc);                                              \
      }                                                                                          \
      __builtin_amdgcn_sched_barrier(0);                                                         \
    }
    ONE_STAGE(0, a, b)
    ONE_STAGE(1, b, a)
#undef ONE_STAGE
    // partial tiles meet in LDS: element e = 4 lane + i is (row 4 (lane / 16) + i, column lane % 16)
    float* rp = red + par * WV * 256;
    *reinterpret_cast<float4*>(rp + wave * 256 + 4 * lane) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    // each wave sums aligned blocks of 64 elements, so a row's 16 columns
    // (elements 64 (r / 4) + 4 col + r % 4) sit in one wave; the sums and
    // keys stay in LDS until the loop ends (a global store inside the loop
    // made the compiler wait for the whole load ring at every tile)
    for (int e = threadIdx.x; e < 256; e += WV * 64) {
      float z = rp[e];
#pragma unroll
      for (int w = 1; w < WV; ++w) z += rp[w * 256 + e];
      const int le = e >> 2, r = 4 * (le >> 4) + (e & 3), col = le & 15;
      const int v = 16 * (t0 + n) + r;
      const bool ok = v < V;
      zout[n * 256 + col * 16 + r] = z;
      // the row's maximum over the 15 positions: lanes (e & 3) + 4 col
      float m = col < DOMINO_T ? z : -__builtin_huge_valf();
      m = fmaxf(m, __shfl_xor(m, 4, 64));
      m = fmaxf(m, __shfl_xor(m, 8, 64));
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (col == 0) {
        kout[n * 16 + r] = orderable(m);
        if (ok) best0 = umax64(best0, pack_key(z, (uint32_t)v));
      }
    }
    par ^= 1;
  }
#undef ONE_PUT
#undef ONE_LOAD8
  __syncthreads();
  // the workgroup's logits [15, V] and keys: for each position one contiguous
  // range of ids, consecutive threads on consecutive ids
  for (int i = threadIdx.x; i < ntiles * 16 * 16; i += WV * 64) {
    const int r = i & 15, nc = i >> 4, n = nc % ntiles, col = nc / ntiles;
    const int v = 16 * (t0 + n) + r;
    if (v < V) {
      if (col < DOMINO_T) {
        out[(size_t)col * V + v] = zout[n * 256 + col * 16 + r];
      } else if (keys) {
        const uint32_t key = kout[n * 16 + r];
        keys[v] = key;
        if (hist0) atomicAdd(&hloc[key >> 21], 1u);
      }
    }
  }
  if (hist0) {
    __syncthreads();
    for (int i = threadIdx.x; i < 2048; i += WV * 64)
      if (hloc[i]) atomicAdd(&hist0[i], hloc[i]);
  }
  // first proposal: the workgroup's best (value, lowest id), published once
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) best0 = umax64(best0, shfl_xor_u64(best0, m));
  __shared__ uint64_t wbest[WV];
  if (lane == 0) wbest[wave] = best0;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t b = wbest[0];
#pragma unroll
    for (int w = 1; w < WV; ++w) b = umax64(b, wbest[w]);
    publish_slot(slot0, 0, b);
  }
}

size_t one_lds(int wv, int maxt) {
  return (size_t)wv * 8192 + 2 * (size_t)wv * 256 * sizeof(float) +
         (size_t)maxt * (256 + 16) * sizeof(float) + 2048 * sizeof(uint32_t);
}
constexpr size_t kOneLdsLimit = 156 * 1024;  // dynamic LDS (the static part is WV words)

// one workgroup per CU, each a contiguous range of at most maxt tiles
void one_grid(int V, int* grid, int* maxt) {
  const int S = (V + 15) / 16;
  *grid = min(S, cu_count());
  *maxt = (S + *grid - 1) / *grid;
}

template <int WV, int KS>
void one_launch(const uint16_t* W, const uint16_t* X, float* out, uint32_t* keys, uint32_t* hist0,
                uint64_t* slot0, int V, int H, hipStream_t st) {
  int grid, maxt;
  one_grid(V, &grid, &maxt);
  DLAUNCH((lmhead_one_kernel<WV, KS>), dim3(grid), dim3(WV * 64), one_lds(WV, maxt), st,
          (const bf16_t*)W, (const bf16_t*)X, out, keys, hist0, slot0, V, H, maxt);
}

}  // namespace

// compute units of the current device (queried once; the grids sized with it
// only set how work is divided, never what is computed)
int cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
  }
  return cus;
}

// waves per workgroup and k steps per wave for hidden width H (a wave owns
// 512 of K: 64 VGPRs of activations and 64 of one tile's loads)
static void one_shape(int H, int* wv, int* ks) {
  *ks = 16;
  *wv = H / (32 * *ks);
}

bool lmhead_one_supported(int V, int H) {
  if (H % 512) return false;
  int wv, ks, grid, maxt;
  one_shape(H, &wv, &ks);
  one_grid(V, &grid, &maxt);
  return wv >= 2 && wv <= 10 && wv % 2 == 0 && one_lds(wv, maxt) <= kOneLdsLimit;
}

void lmhead_one_prepare() {
#define SET(WV, KS) \
  (void)hipFuncSetAttribute((const void*)lmhead_one_kernel<WV, KS>, \
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kOneLdsLimit)
  SET(2, 16);
  SET(4, 16);
  SET(6, 16);
  SET(8, 16);
  SET(10, 16);
#undef SET
}

void launch_lmhead_one(const uint16_t* W, const uint16_t* X, float* out, uint32_t* keys,
                       uint32_t* hist0, uint64_t* slot0, int V, int H, hipStream_t st) {
  int wv, ks;
  one_shape(H, &wv, &ks);
  switch (wv) {
    case 2: one_launch<2, 16>(W, X, out, keys, hist0, slot0, V, H, st); break;
    case 4: one_launch<4, 16>(W, X, out, keys, hist0, slot0, V, H, st); break;
    case 6: one_launch<6, 16>(W, X, out, keys, hist0, slot0, V, H, st); break;
    case 8: one_launch<8, 16>(W, X, out, keys, hist0, slot0, V, H, st); break;
    default: one_launch<10, 16>(W, X, out, keys, hist0, slot0, V, H, st); break;
  }
}
