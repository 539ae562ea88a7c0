// LM-head GEMM with the block's per-id reductions fused into its epilogue.
//
//   base[t, b, v] = sum_i hidden[b, t, i] * lm_head[v, i]          (stored, step-major)
//   key[b, v]     = orderable(max_t base[t, b, v])                 (pool score, optional)
//   word[b]      := max over v of packed (base[0, b, v], v)         (first proposal)
//
// "Add correctness-first Domino support to DFlash V2" (sglang PR #31328),
// "Design": base projection over the full vocabulary, first proposal = its
// full-vocabulary argmax, one block-shared pool per request built from the
// block's base logits; "feat: support tensor-parallel Domino rollout"
// (sglang PR #32018), "Rollout performance": step-major packing.
//
// Tiling for gfx950: a workgroup computes 256 vocabulary rows x 240 columns,
// the columns being 16 requests x 15 draft positions ordered position-major
// (column t*16 + j is request b0+j at position t).  Four waves each own 64
// rows and all 240 columns: 4 x 15 accumulator tiles (240 AGPRs), 60 MFMAs
// per 32-wide k slice against 19 LDS fragment reads.  Both operands reach
// LDS by direct global->LDS copies (no staging registers, which the 240
// accumulators leave no room for) into a 5-slice ring laid out fragment by
// fragment, so 4 slices are in flight while one is consumed and every
// fragment read is a contiguous, conflict-free 16-byte load per lane.
// Because a lane's
// accumulators hold all 15 positions of its (request, row) pairs, the max
// over the block and the position-0 argmax need no extra pass over memory.
// Workgroups sharing lm_head rows (the request groups of one vocabulary
// tile) are dealt to the same XCD back to back so the rows are fetched into
// that XCD's L2 once.
#include "common.h"
#include "launch.h"

namespace {

constexpr int kBN = 256;             // vocabulary rows per workgroup (16 row tiles)
constexpr int kBJ = 16;              // requests per workgroup
constexpr int kStages = 5;           // LDS ring depth (k slices of 32)
constexpr int kBlocks = kBN / 16 + DOMINO_T;  // 31 fragment blocks per slice
constexpr int kSliceBytes = kBlocks * 1024;

// global -> LDS direct copy of 16 bytes per lane; lane l lands at dst + 16*l
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}
// the same for lm_head: non-temporal, since every line is read once (kept in
// the L2s, it only displaces what later kernels read; 8B K = 2048 blocks at
// 12 and 16 requests 3% faster)
__device__ __forceinline__ void dma16_nt(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 2);
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Epilogue shared by both kernels: store base, the pool score keys and the
// position-0 argmax of the workgroup's 256 rows x 16 requests.
__device__ __forceinline__ void fused_epilogue(const FusedArgs& a, const v4f (&acc)[4][DOMINO_T],
                                               unsigned char* ring, int v0, int b0, int wave,
                                               int row, int q, int tid) {
  const int V = a.V, B = a.B;
  const int b = b0 + row;
  const bool bok = b < B;
  const bool vec = (V & 3) == 0;
  uint64_t best0 = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int v = v0 + wave * 64 + r * 16 + 4 * q;
    const bool full = vec && v + 3 < V;
#pragma unroll
    for (int t = 0; t < DOMINO_T; ++t) {
      if (!bok) break;
      float* o = a.base + ((size_t)t * B + b) * V + v;
      if (full) {
        *reinterpret_cast<float4*>(o) = make_float4(acc[r][t][0], acc[r][t][1], acc[r][t][2], acc[r][t][3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v + i < V) o[i] = acc[r][t][i];
      }
    }
    uint32_t kk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = acc[r][0][i];
#pragma unroll
      for (int t = 1; t < DOMINO_T; ++t) m = fmaxf(m, acc[r][t][i]);
      kk[i] = orderable(m);
      const uint64_t k0 = pack_key(acc[r][0][i], (uint32_t)(v + i));
      best0 = (v + i < V) ? umax64(best0, k0) : best0;
    }
    if (a.keys && bok) {
      uint32_t* kp = a.keys + (size_t)b * V + v;
      if (full) {
        *reinterpret_cast<uint4*>(kp) = make_uint4(kk[0], kk[1], kk[2], kk[3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v + i < V) kp[i] = kk[i];
      }
    }
  }
  // first proposal: lanes row, row+16, row+32, row+48 hold request b
  best0 = umax64(best0, shfl_xor_u64(best0, 16));
  best0 = umax64(best0, shfl_xor_u64(best0, 32));
  uint64_t (*wb)[16] = reinterpret_cast<uint64_t (*)[16]>(ring);
  if (q == 0) wb[wave][row] = best0;
  __syncthreads();
  if (tid < 16 && b0 + tid < B)
    publish_slot(a.slots, b0 + tid,
                umax64(umax64(wb[0][tid], wb[1][tid]), umax64(wb[2][tid], wb[3][tid])));
}

__global__ __launch_bounds__(256) void lmhead_fused_kernel(FusedArgs a) {
  const int V = a.V, H = a.H, B = a.B;
  const int nvt = (V + kBN - 1) / kBN, ngrp = (B + kBJ - 1) / kBJ;
  const int j = blockIdx.x, xcd = j & 7, local = j >> 3;
  const int vt = (local / ngrp) * 8 + xcd, grp = local % ngrp;
  if (vt >= nvt) return;  // uniform per workgroup, before any barrier
  const int v0 = vt * kBN, b0 = grp * kBJ;

  // Ring of kStages k-slices.  Slice layout: 31 blocks of 1 KB, block i < 16
  // = lm_head rows v0 + 16i .. +15, block 16 + t = the 16 requests at draft
  // position t; inside a block lane l's 16 bytes sit at 16*l and are exactly
  // that lane's MFMA fragment (row/column l % 16, k = 8 * (l / 16) .. +7).
  extern __shared__ __align__(1024) unsigned char ring[];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;

  // this wave's copy duties per slice: A blocks wave*4 .. +3 and B blocks
  // t = wave, wave+4, wave+8, wave+12 (< 15) -> 8 copies (7 for wave 3)
  const char* const Wb = reinterpret_cast<const char*>(a.W);
  const char* const Xb = reinterpret_cast<const char*>(a.X);
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    aoff[i] = ((uint32_t)min(v0 + (wave * 4 + i) * 16 + row, V - 1) * (uint32_t)H + q * 8) * 2u;
    const int t = min(wave + 4 * i, DOMINO_T - 1);
    boff[i] = (((uint32_t)min(b0 + row, B - 1) * DOMINO_T + t) * (uint32_t)H + q * 8) * 2u;
  }
  const bool four_b = wave + 12 < DOMINO_T;  // waves 0..2 copy 4 B blocks
  auto issue = [&](int s) {
    unsigned char* slot = ring + (s % kStages) * kSliceBytes;
    const uint32_t kb = (uint32_t)s * 64u;  // 32 bf16 per slice
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_nt(Wb + (aoff[i] + kb), slot + (wave * 4 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 3; ++i) dma16(Xb + (boff[i] + kb), slot + (16 + wave + 4 * i) * 1024);
    if (four_b) dma16(Xb + (boff[3] + kb), slot + (16 + wave + 12) * 1024);
  };

  v4f acc[4][DOMINO_T];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < DOMINO_T; ++t) acc[r][t] = zero4();

  const int nk = H / 32;
  for (int s = 0; s < kStages - 1 && s < nk; ++s) issue(s);
  for (int s = 0; s < nk; ++s) {
    // slice s has landed for this wave once at most kStages-2 newer slices
    // are still in flight; the barrier then covers every wave's copies
    if (s + kStages - 2 < nk) {
      if (four_b) wait_vm<8 * (kStages - 2)>();
      else wait_vm<7 * (kStages - 2)>();
    } else {
      wait_vm<0>();
    }
    lds_barrier();
    // every wave has finished slice s-1: its slot takes slice s + kStages - 1
    if (s + kStages - 1 < nk) issue(s + kStages - 1);
    const unsigned char* slot = ring + (s % kStages) * kSliceBytes + lane * 16;
    v8s af[4], bf[DOMINO_T];
#pragma unroll
    for (int r = 0; r < 4; ++r) af[r] = *reinterpret_cast<const v8s*>(slot + (wave * 4 + r) * 1024);
#pragma unroll
    for (int t = 0; t < DOMINO_T; ++t) bf[t] = *reinterpret_cast<const v8s*>(slot + (16 + t) * 1024);
#pragma unroll
    for (int t = 0; t < DOMINO_T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r][t] = mfma_bf16(af[r], bf[t], acc[r][t]);
  }
  lds_barrier();  // the ring is free again

  fused_epilogue(a, acc, ring, v0, b0, wave, row, q, tid);
}

// Line-copy kernel with separate operand rings.  A direct global->LDS copy
// moves fastest when its 64 lanes cover whole 128-byte lines (8 rows x 128 B
// per instruction run at about four times the rate of the 16 rows x 64 B of
// an MFMA fragment on gfx950), so a stage holds 64 k and every 1 KB block is
// 8 rows x 64 bf16.  Within a row the 16-byte chunk of logical index c sits
// at position c ^ (r16 >> 1), r16 being the row's index in its 16-row tile,
// which keeps the 16 lanes of a fragment read on distinct banks.  lm_head
// rows come from HBM, so their ring is three stages deep (two in flight);
// the activations are cache resident and double-buffered.  Each iteration
// issues the activation copies of stage s + 1 before the lm_head copies of
// stage s + 2, so "all but this wave's newest 8 copies have landed" covers
// both operands of stage s + 1 at the next iteration.
constexpr int kStageK = 64;
constexpr int kABlocks = kBN / 8;                  // 32 blocks of 8 lm_head rows
constexpr int kBBlocks = 2 * DOMINO_T;             // 30 blocks of 8 requests at one position
constexpr int kARing = 3, kBRing = 2;
static_assert(kARing + kBRing == 5 && (kARing == 2 || kARing == 3), "ring depths");
constexpr bool kADeep = kARing > kBRing;  // which operand runs two stages ahead
constexpr int kReadWindow = 8;  // fragment reads kept ahead of the products
constexpr int kAStage = kABlocks * 1024, kBStage = kBBlocks * 1024;
constexpr size_t kLinesLds = (size_t)kARing * kAStage + (size_t)kBRing * kBStage;  // 154-156 KB
constexpr int kACopies = kABlocks / 4;             // 8 per wave
constexpr int kBCopies = (kBBlocks + 3) / 4;       // 8 (7 for waves 2, 3)

__global__ __launch_bounds__(256) void lmhead_lines_kernel(FusedArgs a) {
  const int V = a.V, H = a.H, B = a.B;
  const int nvt = (V + kBN - 1) / kBN, ngrp = (B + kBJ - 1) / kBJ;
  const int j = blockIdx.x, xcd = j & 7, local = j >> 3;
  const int vt = (local / ngrp) * 8 + xcd, grp = local % ngrp;
  if (vt >= nvt) return;  // uniform per workgroup, before any barrier
  const int v0 = vt * kBN, b0 = grp * kBJ;
  extern __shared__ __align__(1024) unsigned char ring[];
  unsigned char* const aring = ring;
  unsigned char* const bring = ring + kARing * kAStage;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;

  // copy duties: A blocks wave + 4i (i < 8), B blocks wave + 4i (< 30); lane
  // (rr = lane / 8, p = lane % 8) fetches logical chunk p ^ (r16 >> 1) of row
  // rr of its block
  const char* const Wb = reinterpret_cast<const char*>(a.W);
  const char* const Xb = reinterpret_cast<const char*>(a.X);
  const int rr = lane >> 3, pp = lane & 7;
  uint32_t aoff[kACopies], boff[kBCopies];
#pragma unroll
  for (int i = 0; i < kACopies; ++i) {
    const int blk = wave + 4 * i;
    const int r16 = (blk & 1) * 8 + rr;
    const int v = min(v0 + blk * 8 + rr, V - 1);
    aoff[i] = ((uint32_t)v * (uint32_t)H + (pp ^ (r16 >> 1)) * 8) * 2u;
  }
#pragma unroll
  for (int i = 0; i < kBCopies; ++i) {
    const int blk = min(wave + 4 * i, kBBlocks - 1);
    const int r16 = (blk & 1) * 8 + rr;
    const int t = blk >> 1;
    const int bb = min(b0 + r16, B - 1);
    boff[i] = (((uint32_t)bb * DOMINO_T + t) * (uint32_t)H + (pp ^ (r16 >> 1)) * 8) * 2u;
  }
  const bool eight_b = wave + 4 * (kBCopies - 1) < kBBlocks;
  auto issue_a = [&](int s) {
    unsigned char* slot = aring + (s % kARing) * kAStage;
    const uint32_t kb = (uint32_t)s * (kStageK * 2);
#pragma unroll
    for (int i = 0; i < kACopies; ++i) dma16_nt(Wb + (aoff[i] + kb), slot + (wave + 4 * i) * 1024);
  };
  auto issue_b = [&](int s) {
    unsigned char* slot = bring + (s % kBRing) * kBStage;
    const uint32_t kb = (uint32_t)s * (kStageK * 2);
#pragma unroll
    for (int i = 0; i < kBCopies - 1; ++i) dma16(Xb + (boff[i] + kb), slot + (wave + 4 * i) * 1024);
    if (eight_b)
      dma16(Xb + (boff[kBCopies - 1] + kb), slot + (wave + 4 * (kBCopies - 1)) * 1024);
  };

  v4f acc[4][DOMINO_T];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < DOMINO_T; ++t) acc[r][t] = zero4();

  // fragment of this lane inside a block pair (16 rows): block 2T + (row >> 3),
  // row (row & 7), chunk (h * 4 + q) ^ (row >> 1)
  const int frag0 = (row >> 3) * 1024 + (row & 7) * 128;
  const int sw = row >> 1;
  const int ns = H / kStageK;
  // prologue: the shallow operand's stage 0, then the deep one's stages 0, 1
  // in the order the loop keeps (deep copies of the farthest stage newest)
  if (kADeep) {
    issue_a(0);
    issue_b(0);
    if (ns > 1) issue_a(1);
  } else {
    issue_b(0);
    issue_a(0);
    if (ns > 1) issue_b(1);
  }
  for (int s = 0; s < ns; ++s) {
    // this wave's newest copies are the deep operand's stage s + 1 (if any)
    if (s + 1 < ns) {
      if (kADeep) wait_vm<kACopies>();
      else if (eight_b) wait_vm<kBCopies>();
      else wait_vm<kBCopies - 1>();
    } else {
      wait_vm<0>();
    }
    lds_barrier();  // everyone's copies of stage s landed; stage s - 1 is consumed
    if (kADeep) {
      if (s + 1 < ns) issue_b(s + 1);
      if (s + 2 < ns) issue_a(s + 2);
    } else {
      if (s + 1 < ns) issue_a(s + 1);
      if (s + 2 < ns) issue_b(s + 2);
    }
    const unsigned char* as = aring + (s % kARing) * kAStage + frag0;
    const unsigned char* bs = bring + (s % kBRing) * kBStage + frag0;
    // The stage's 38 fragment reads (A then B of the first 32-wide half, then
    // of the second) run as one stream kReadWindow reads ahead of the 30
    // product steps (4 MFMAs against one B fragment each).  Fewer than 16
    // reads are ever outstanding, so every wait names exactly the fragment
    // it needs; the scheduling barriers keep that order.
    constexpr int kFrags = 2 * (4 + DOMINO_T);
    v8s fr[kFrags];
    auto rd = [&](int k) {
      const int h = k / (4 + DOMINO_T), idx = k % (4 + DOMINO_T);
      const int cofs = ((h * 4 + q) ^ sw) * 16;
      fr[k] = idx < 4 ? *reinterpret_cast<const v8s*>(as + 2 * (wave * 4 + idx) * 1024 + cofs)
                      : *reinterpret_cast<const v8s*>(bs + 2 * (idx - 4) * 1024 + cofs);
    };
    int issued = 0;
#pragma unroll
    for (int jstep = 0; jstep < 2 * DOMINO_T; ++jstep) {
      const int h = jstep / DOMINO_T, t = jstep % DOMINO_T;
      const int need = h * (4 + DOMINO_T) + 4 + t;
      const int upto = min(need + kReadWindow, kFrags - 1);
#pragma unroll
      for (int k = 0; k < kFrags; ++k)
        if (k >= issued && k <= upto) rd(k);
      issued = max(issued, upto + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[r][t] = mfma_bf16(fr[h * (4 + DOMINO_T) + r], fr[need], acc[r][t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();  // the rings are free again
  fused_epilogue(a, acc, ring, v0, b0, wave, row, q, tid);
}

// ------------------------------------------------- 32x32x16 matrix products
// 9 to 24 requests (and up to 8 when H is not a multiple of 128, which the
// vocabulary-range kernel below needs).
//
// A workgroup computes 256 vocabulary rows against 8 requests x 16 draft
// positions (position 15 is padding: its rows repeat position 14 and are
// dropped).  The activation rows are the A operand and the lm_head rows the
// B operand of V_MFMA_F32_32X32X16_BF16, so lane l of an output tile holds
// vocabulary id l % 32 and 16 activation rows 8 (i / 4) + 4 (l / 32) + i % 4:
// each request's positions sit in one lane pair (l, l + 32), a base-logit
// store writes two whole 128-byte lines, the block max of a (request, id) is
// one shuffle away and position 0 is register 0 / 8 of lanes 0..31.  Each of
// the four waves owns 64 vocabulary rows and all 128 activation rows (4 x 2
// tiles, 128 accumulators).  Operands reach LDS as the line kernel's: 8 rows
// x 128 B per copy, 64-wide k stages, 16-byte chunk c of a row at position
// c ^ ((r >> 1) & 7) (r = the row's index in its 32-row tile), so the 16
// lanes of a fragment read hit distinct banks; both rings are three stages
// deep (two in flight, 144 KB).
//
// Measured against the line kernel at 8B shapes (LM-head ms): B = 5 0.344 /
// 0.396, 8 0.363 / 0.413, 16 0.431 / 0.458, 24 0.652 / 0.661, 32 0.838 /
// 0.668, 48 1.187 / 0.975.  Its loop alone (no copies) runs at ~1 PFLOP/s: the
// compiler waits for all outstanding LDS reads twice per stage and one wave
// per SIMD cannot cover those stalls, so above 24 requests the line kernel's
// higher fragment reuse wins.
typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int kM32MaxBatch = 24;
constexpr int kMR = 8;                         // requests per workgroup
constexpr int kMRows = kMR * 16;               // activation rows per workgroup
constexpr int kMK = 64;                        // k per stage
constexpr int kMXStage = kMRows * kMK * 2;     // 16 KB
constexpr int kMXCopies = kMRows / 8 / 4;      // 4 per wave
constexpr int kMWindow = 6;                    // fragment reads ahead of the products
// TV vocabulary tiles of 32 rows per wave (workgroup: 128 TV rows); ring
// depth R stages per operand
template <int TV>
struct M32 {
  static constexpr int kMV = 128 * TV;
  static constexpr int kR = TV == 2 ? 3 : 4;
  static constexpr int kVStage = kMV * kMK * 2;
  static constexpr size_t kLds = (size_t)kR * (kVStage + kMXStage);  // 144 / 128 KB
  static constexpr int kVCopies = kMV / 8 / 4;
};

__device__ __forceinline__ v16f mfma32(v8s a, v8s b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int TV>
__global__ __launch_bounds__(256) void lmhead_m32_kernel(FusedArgs a) {
  using C = M32<TV>;
  constexpr int kMV = C::kMV, kMRing = C::kR, kMVStage = C::kVStage, kMVCopies = C::kVCopies;
  const int V = a.V, H = a.H, B = a.B;
  const int nvt = (V + kMV - 1) / kMV, ngrp = (B + kMR - 1) / kMR;
  const int j = blockIdx.x, xcd = j & 7, local = j >> 3;
  const int vt = (local / ngrp) * 8 + xcd, grp = local % ngrp;
  if (vt >= nvt) return;  // uniform per workgroup, before any barrier
  const int v0 = vt * kMV, b0 = grp * kMR;
  extern __shared__ __align__(1024) unsigned char ring[];
  unsigned char* const wring = ring;
  unsigned char* const xring = ring + kMRing * kMVStage;
  const int lane = threadIdx.x & 63, wave = wave_index();

  // copy duties: lm_head blocks wave + 4i (i < kMVCopies) and activation
  // blocks wave + 4i (i < 4) of 8 rows; lane (rr = lane / 8, pp = lane % 8)
  // fetches logical chunk pp ^ ((r >> 1) & 7) of row rr of its block
  const char* const Wb = reinterpret_cast<const char*>(a.W);
  const char* const Xb = reinterpret_cast<const char*>(a.X);
  const int rr = lane >> 3, pp = lane & 7;
  uint32_t woff[kMVCopies], xoff[kMXCopies];
#pragma unroll
  for (int i = 0; i < kMVCopies; ++i) {
    const int blk = wave + 4 * i;
    const int r = (blk & 3) * 8 + rr;
    const int v = min(v0 + blk * 8 + rr, V - 1);
    woff[i] = ((uint32_t)v * (uint32_t)H + (uint32_t)(pp ^ ((r >> 1) & 7)) * 8u) * 2u;
  }
#pragma unroll
  for (int i = 0; i < kMXCopies; ++i) {
    const int blk = wave + 4 * i;
    const int R = blk * 8 + rr;  // activation row of the workgroup
    const int r = R & 31;
    const int req = min(b0 + (R >> 4), B - 1);
    const int pos = min(R & 15, DOMINO_T - 1);
    xoff[i] = (((uint32_t)req * DOMINO_T + (uint32_t)pos) * (uint32_t)H +
               (uint32_t)(pp ^ ((r >> 1) & 7)) * 8u) * 2u;
  }
  auto issue = [&](int s) {
    unsigned char* ws = wring + (s % kMRing) * kMVStage;
    unsigned char* xs = xring + (s % kMRing) * kMXStage;
    const uint32_t kb = (uint32_t)s * (kMK * 2);
#pragma unroll
    for (int i = 0; i < kMVCopies; ++i) dma16_nt(Wb + (woff[i] + kb), ws + (wave + 4 * i) * 1024);
#pragma unroll
    for (int i = 0; i < kMXCopies; ++i) dma16(Xb + (xoff[i] + kb), xs + (wave + 4 * i) * 1024);
  };

  v16f acc[4][TV];
#pragma unroll
  for (int ta = 0; ta < 4; ++ta)
#pragma unroll
    for (int tv = 0; tv < TV; ++tv)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[ta][tv][i] = 0.f;

  // fragment of this lane in a 32-row tile: row lane % 32, chunk 2 k16 + lane / 32
  const int frow = lane & 31, fhi = lane >> 5, fsw = (frow >> 1) & 7;
  const int ns = H / kMK;
#pragma unroll
  for (int p = 0; p < kMRing - 1; ++p)
    if (p < ns) issue(p);
  for (int s = 0; s < ns; ++s) {
    // this wave's newest copies are the stages after s (up to kMRing - 2 of them)
    const int ahead = min(ns - 1 - s, kMRing - 2);
    if (ahead >= 2) wait_vm<2 * (kMVCopies + kMXCopies)>();
    else if (ahead == 1) wait_vm<kMVCopies + kMXCopies>();
    else wait_vm<0>();
    lds_barrier();  // everyone's stage s landed; stage s - 1 is consumed
    if (s + kMRing - 1 < ns) issue(s + kMRing - 1);
    const unsigned char* wsb = wring + (s % kMRing) * kMVStage + wave * (TV * 4096) + frow * 128;
    const unsigned char* xsb = xring + (s % kMRing) * kMXStage + frow * 128;
    // The stage's fragment reads (per 16-wide k step: TV lm_head, then 4
    // activation fragments) run as one stream kMWindow reads ahead of the
    // products; the scheduling barriers keep it.
    constexpr int kPer = TV + 4;
    constexpr int kF = kPer * (kMK / 16);
    v8s fr[kF];
    auto rd = [&](int k) {
      const int k16 = k / kPer, idx = k % kPer;
      const int cofs = ((2 * k16 + fhi) ^ fsw) * 16;
      fr[k] = idx < TV ? *reinterpret_cast<const v8s*>(wsb + idx * 4096 + cofs)
                       : *reinterpret_cast<const v8s*>(xsb + (idx - TV) * 4096 + cofs);
    };
    int issued = 0;
#pragma unroll
    for (int k16 = 0; k16 < kMK / 16; ++k16) {
      const int upto = min(k16 * kPer + kPer - 1 + kMWindow, kF - 1);
#pragma unroll
      for (int k = 0; k < kF; ++k)
        if (k >= issued && k <= upto) rd(k);
      issued = max(issued, upto + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ta = 0; ta < 4; ++ta)
#pragma unroll
        for (int tv = 0; tv < TV; ++tv)
          acc[ta][tv] = mfma32(fr[k16 * kPer + TV + ta], fr[k16 * kPer + tv], acc[ta][tv]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: base logits (step-major), pool score keys, first-proposal argmax
  const int vl = lane & 31, hh = lane >> 5;
  uint64_t best[kMR];
#pragma unroll
  for (int r = 0; r < kMR; ++r) best[r] = 0;
#pragma unroll
  for (int ta = 0; ta < 4; ++ta)
#pragma unroll
    for (int tv = 0; tv < TV; ++tv) {
      const int v = v0 + wave * (TV * 32) + tv * 32 + vl;
      const bool vok = v < V;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int req = b0 + 2 * ta + jj;
        const bool ok = vok && req < B;
        float m = -INFINITY;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int i = jj * 8 + ii;
          const int pos = 8 * ((i >> 2) & 1) + 4 * hh + (i & 3);
          const float y = acc[ta][tv][i];
          if (pos < DOMINO_T) {
            m = fmaxf(m, y);
            if (ok) a.base[((size_t)pos * B + req) * V + v] = y;
          }
        }
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (a.keys && hh == 0 && ok) a.keys[(size_t)req * V + v] = orderable(m);
        const uint64_t k0 = pack_key(acc[ta][tv][jj * 8], (uint32_t)v);  // position 0 on hh == 0
        best[2 * ta + jj] = (hh == 0 && vok) ? umax64(best[2 * ta + jj], k0) : best[2 * ta + jj];
      }
    }
#pragma unroll
  for (int r = 0; r < kMR; ++r) best[r] = wave_max_u64(best[r]);
  __shared__ uint64_t wb[4][kMR];
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < kMR; ++r) wb[wave][r] = best[r];
  __syncthreads();
  if (threadIdx.x < kMR && b0 + (int)threadIdx.x < B) {
    const int r = threadIdx.x;
    publish_slot(a.slots, b0 + r, umax64(umax64(wb[0][r], wb[1][r]), umax64(wb[2][r], wb[3][r])));
  }
}

// One 64-wide k stage of the m32 products from LDS: per 16-wide k step TV
// lm_head and 4 activation fragments, read as one stream kMWindow reads
// ahead of the products (the scheduling barriers keep it).
template <int TV>
__device__ __forceinline__ void m32_products(const unsigned char* wsb, const unsigned char* xsb,
                                             int fhi, int fsw, v16f (&acc)[4][TV]) {
  constexpr int kPer = TV + 4;
  constexpr int kF = kPer * (kMK / 16);
  v8s fr[kF];
  int issued = 0;
#pragma unroll
  for (int k16 = 0; k16 < kMK / 16; ++k16) {
    const int upto = min(k16 * kPer + kPer - 1 + kMWindow, kF - 1);
#pragma unroll
    for (int k = 0; k < kF; ++k)
      if (k >= issued && k <= upto) {
        const int kk = k / kPer, idx = k % kPer;
        const int cofs = ((2 * kk + fhi) ^ fsw) * 16;
        fr[k] = idx < TV ? *reinterpret_cast<const v8s*>(wsb + idx * 4096 + cofs)
                         : *reinterpret_cast<const v8s*>(xsb + (idx - TV) * 4096 + cofs);
      }
    issued = max(issued, upto + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int tv = 0; tv < TV; ++tv)
        acc[ta][tv] = mfma32(fr[k16 * kPer + TV + ta], fr[k16 * kPer + tv], acc[ta][tv]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Epilogue of one chunk of the range kernel (requests 0..7, the wave's TV
// tiles from vocabulary row vw): pool score keys, the lane's running
// position-0 argmax per request and the base logits; clears the
// accumulators.  A lane holds positions 4 hh + {0, 1, 2, 3, 8, 9, 10, 11} of
// its (request, id): one guarded run of stores at fixed position strides per
// request, position 15 (the padding row, hh = 1) never stored.
template <int TV, bool KEEP>
__device__ __forceinline__ void range_epilogue(const FusedArgs& a, v16f (&acc)[4][TV], int vw,
                                               int rend, int vl, int hh,
                                               uint64_t (&best)[kMR]) {
  // opaque copies, so the store addresses are formed here and not hoisted
  // out of the stage loop (where they would hold some 200 registers)
  int V = a.V, B = a.B;
  asm volatile("" : "+s"(V), "+s"(B));
  const size_t pstride = (size_t)B * V;  // elements from one position to the next
#pragma unroll
  for (int ta = 0; ta < 4; ++ta)
#pragma unroll
    for (int tv = 0; tv < TV; ++tv) {
      const int v = vw + tv * 32 + vl;
      const bool vok = v < rend;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int req = 2 * ta + jj;
        const bool ok = vok && req < B;
        if (a.keys) {
          float m = acc[ta][tv][jj * 8];
#pragma unroll
          for (int ii = 1; ii < 7; ++ii) m = fmaxf(m, acc[ta][tv][jj * 8 + ii]);
          if (hh == 0) m = fmaxf(m, acc[ta][tv][jj * 8 + 7]);
          m = fmaxf(m, __shfl_xor(m, 32, 64));
          if (hh == 0 && ok) a.keys[(size_t)req * V + v] = orderable(m);
        }
        const uint64_t k0 = pack_key(acc[ta][tv][jj * 8], (uint32_t)v);  // position 0 on hh == 0
        best[req] = (hh == 0 && vok) ? umax64(best[req], k0) : best[req];
        // Full-vocabulary runs store the logits non-temporally: each
        // correction step streams one whole row of them, and cached rows
        // only displace fc2 (8B, 8 requests: LM-head 1-4 us faster, K0 block
        // 1.131 against 1.145 ms cached).  A pool run (KEEP) reads them back
        // only at its pool ids, which then hit the caches more often when the
        // stores are cached (K = 2048 block 0.528 against 0.524 ms cached).
        // The choice is a template parameter: with a runtime branch the
        // compiler merged the two stores and dropped the non-temporal hint.
        if (ok) {
          float* o = a.base + (size_t)req * V + v + (size_t)(4 * hh) * pstride;
          if constexpr (KEEP) {
#pragma unroll
            for (int ii = 0; ii < 7; ++ii) o[(size_t)(8 * (ii >> 2) + (ii & 3)) * pstride] = acc[ta][tv][jj * 8 + ii];
            if (hh == 0) o[11 * pstride] = acc[ta][tv][jj * 8 + 7];
          } else {
#pragma unroll
            for (int ii = 0; ii < 7; ++ii)
              __builtin_nontemporal_store(acc[ta][tv][jj * 8 + ii],
                                          &o[(size_t)(8 * (ii >> 2) + (ii & 3)) * pstride]);
            if (hh == 0) __builtin_nontemporal_store(acc[ta][tv][jj * 8 + 7], &o[11 * pstride]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[ta][tv][i] = 0.f;
    }
}

// Up to 8 requests: vocabulary ranges, producer and consumer waves.
//
// One workgroup per compute unit owns a contiguous range of 32-row vocabulary
// tiles (ranges differ by at most one tile, so every CU streams the same
// share of lm_head; a grid of 128-row tiles leaves part of the chip idle in
// its last round) and walks it in chunks of 4 TV tiles with the m32
// kernel's products, LDS layout and epilogue.  Waves 4..7 produce: they
// stage both operands through registers (a load-only probe streamed
// lm_head-shaped rows at 1.8-3.7 TB/s through direct global->LDS copies,
// 6.1 TB/s through registers) into two LDS slots.  Waves 0..3 consume: each
// owns TV tiles of a chunk against all 8 requests and takes one stage's
// products from LDS per barrier, so the matrix cores work while the
// producers' loads are in flight.  (With every wave doing both, a stage's products and loads ran one
// after the other: 8B B = 8 338 against 279 us.)  The chunks form one flat
// sequence of stages, so the next chunk's first stages are loading during a
// chunk's epilogue.
// Rows past the range (the last chunk's missing tiles) re-read the range's
// first row, an L2 hit, instead of branching around the load.  Each
// consumer lane keeps its position-0 maxima across chunks; the workgroup
// publishes one word per request at the end.
template <int TV, bool KEEP>
__global__ __launch_bounds__(512) void lmhead_range_kernel(FusedArgs a) {
  using C = M32<TV>;
  constexpr int kMV = C::kMV, kMVStage = C::kVStage, kMVCopies = C::kVCopies;
  const int V = a.V, H = a.H, B = a.B;
  const int nt = (V + 31) / 32, G = gridDim.x, g = blockIdx.x;
  const int t0 = (int)((long long)g * nt / G), t1 = (int)((long long)(g + 1) * nt / G);
  if (t1 <= t0) return;  // uniform per workgroup, before any barrier
  const int r0 = t0 * 32, rend = min(t1 * 32, V);
  const int nchunk = (t1 - t0 + 4 * TV - 1) / (4 * TV);
  const int ns = H / kMK, nq = nchunk * ns;
  extern __shared__ __align__(1024) unsigned char ring[];
  unsigned char* const wring = ring;
  unsigned char* const xring = ring + 2 * kMVStage;
  const int lane = threadIdx.x & 63, wave = wave_index(), w4 = wave & 3;
  __shared__ uint64_t wb[4][kMR];  // each consumer wave's position-0 maxima

  if (wave >= 4) {
    // ---- producer wave w4: lm_head blocks w4 + 4i of 8 chunk rows and
    // activation blocks w4 + 4i of 8 rows; lane (rr, pp) fetches logical
    // 16-byte chunk pp ^ ((r >> 1) & 7) of row rr of its block
    const int rr = lane >> 3, pp = lane & 7;
    const u32x4* const Wv = reinterpret_cast<const u32x4*>(a.W);
    const u32x4* const Xv = reinterpret_cast<const u32x4*>(a.X);
    const uint32_t hrow = (uint32_t)H / 8;  // 16-byte units per row
    uint32_t wsc[kMVCopies], xoff[kMXCopies];
#pragma unroll
    for (int i = 0; i < kMVCopies; ++i) {
      const int r = ((w4 + 4 * i) & 3) * 8 + rr;
      wsc[i] = (uint32_t)(pp ^ ((r >> 1) & 7));
    }
#pragma unroll
    for (int i = 0; i < kMXCopies; ++i) {
      const int R = (w4 + 4 * i) * 8 + rr;  // activation row of the group
      const int req = min(R >> 4, B - 1);
      const int pos = min(R & 15, DOMINO_T - 1);
      xoff[i] = ((uint32_t)req * DOMINO_T + (uint32_t)pos) * hrow + (uint32_t)(pp ^ (((R & 31) >> 1) & 7));
    }
    // stage Q (clamped to the last: those loads refill a set nobody reads);
    // lm_head non-temporal (read once: 8B B = 8 LM-head 265 -> 258 us, the
    // pool cell's block 0.554 -> 0.525 ms), the activations cached (re-read
    // for every chunk)
#define RANGE_LOAD_W(RW, Q)                                                         \
  {                                                                                 \
    const int q_ = min((Q), nq - 1), c_ = q_ / ns, s_ = q_ - c_ * ns;               \
    const int rc_ = r0 + c_ * kMV + rr;                                             \
    _Pragma("unroll") for (int i = 0; i < kMVCopies; ++i) {                         \
      const int v_ = rc_ + (w4 + 4 * i) * 8;                                        \
      RW[i] = __builtin_nontemporal_load(                                           \
          &Wv[(uint32_t)(v_ < rend ? v_ : r0) * hrow + wsc[i] + 8u * s_]);           \
    }                                                                               \
  }
#define RANGE_LOAD_X(RX, Q)                                                         \
  {                                                                                 \
    const int q_ = min((Q), nq - 1), s_ = q_ % ns;                                  \
    _Pragma("unroll") for (int i = 0; i < kMXCopies; ++i) RX[i] = Xv[xoff[i] + 8u * s_]; \
  }
#define RANGE_PUT(RW, RX, SLOT)                                                     \
  {                                                                                 \
    unsigned char* ws_ = wring + (SLOT) * kMVStage + lane * 16;                     \
    unsigned char* xs_ = xring + (SLOT) * kMXStage + lane * 16;                     \
    _Pragma("unroll") for (int i = 0; i < kMVCopies; ++i)                           \
      *reinterpret_cast<u32x4*>(ws_ + (w4 + 4 * i) * 1024) = RW[i];                 \
    _Pragma("unroll") for (int i = 0; i < kMXCopies; ++i)                           \
      *reinterpret_cast<u32x4*>(xs_ + (w4 + 4 * i) * 1024) = RX[i];                 \
  }
    if constexpr (TV == 1) {
      // Three lm_head register sets (two activation sets): while the
      // consumers take stage Q from slot Q % 2, a step loads the activations
      // of stage Q + 2 and the lm_head rows of stage Q + 3, in that order,
      // then puts stage Q + 1 into the other slot (its stage Q - 1 was
      // finished before the last barrier), so the wait for stage Q + 1 leaves
      // the lm_head loads of stages Q + 2 and Q + 3 in flight.  Six steps
      // cover both set rotations; a step runs only when every earlier one
      // did.  8B LM-head us on one box, three / two sets: B = 2 230-247 /
      // 238-255, 3 234-237 / 243, 4 237-238 / 246.  (At TV = 3 a third set
      // does not fit the registers: the producers spilled loaded data and
      // B = 8 took 401 against 266 us.)
      u32x4 W0[kMVCopies], W1[kMVCopies], W2[kMVCopies], X0[kMXCopies], X1[kMXCopies];
      RANGE_LOAD_W(W0, 0)
      RANGE_LOAD_X(X0, 0)
      RANGE_LOAD_W(W1, 1)
      RANGE_LOAD_X(X1, 1)
      RANGE_LOAD_W(W2, 2)
      RANGE_PUT(W0, X0, 0)
      __syncthreads();
#define RANGE_STEP(I, LX, LW, PW, PX, SLOT)                                         \
  if (q + (I) >= nq) break;                                                       \
  RANGE_LOAD_X(LX, q + (I) + 2)                                                   \
  RANGE_LOAD_W(LW, q + (I) + 3)                                                   \
  __builtin_amdgcn_sched_barrier(0); /* the loads go out before the wait */       \
  RANGE_PUT(PW, PX, SLOT)                                                         \
  __syncthreads();
      for (int q = 0; q < nq; q += 6) {
        RANGE_STEP(0, X0, W0, W1, X1, 1)
        RANGE_STEP(1, X1, W1, W2, X0, 0)
        RANGE_STEP(2, X0, W2, W0, X1, 1)
        RANGE_STEP(3, X1, W0, W1, X0, 0)
        RANGE_STEP(4, X0, W1, W2, X1, 1)
        RANGE_STEP(5, X1, W2, W0, X0, 0)
      }
#undef RANGE_STEP
    } else {
      // two register sets: in the stage that the consumers take from one
      // slot, stage Q + 1 (set B, loaded one stage earlier) goes into the
      // other slot, whose stage Q - 1 they finished before the last barrier,
      // and stage Q + 2 into set A, whose stage Q is in LDS
      u32x4 AW[kMVCopies], AX[kMXCopies], BW[kMVCopies], BX[kMXCopies];
      RANGE_LOAD_W(AW, 0)
      RANGE_LOAD_X(AX, 0)
      RANGE_LOAD_W(BW, 1)
      RANGE_LOAD_X(BX, 1)
      RANGE_PUT(AW, AX, 0)
      __syncthreads();
      for (int q = 0; q < nq; q += 2) {  // nq is even
        RANGE_LOAD_W(AW, q + 2)
        RANGE_LOAD_X(AX, q + 2)
        __builtin_amdgcn_sched_barrier(0);  // the loads go out before the wait for the other set
        RANGE_PUT(BW, BX, 1)
        __syncthreads();
        RANGE_LOAD_W(BW, q + 3)
        RANGE_LOAD_X(BX, q + 3)
        __builtin_amdgcn_sched_barrier(0);
        RANGE_PUT(AW, AX, 0)
        __syncthreads();
      }
    }
#undef RANGE_PUT
#undef RANGE_LOAD_X
#undef RANGE_LOAD_W
    wait_vm<0>();  // the clamped loads past the last stage
    __syncthreads();
  } else {
    // ---- consumer wave w4: vocabulary tiles w4 TV .. w4 TV + TV - 1 of each
    // chunk against all 8 requests
    uint64_t best[kMR];
#pragma unroll
    for (int r = 0; r < kMR; ++r) best[r] = 0;
    v16f acc[4][TV];
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int tv = 0; tv < TV; ++tv)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[ta][tv][i] = 0.f;
    const int frow = lane & 31, fhi = lane >> 5, fsw = (frow >> 1) & 7;
    const unsigned char* const wsb = wring + w4 * (TV * 4096) + frow * 128;
    const unsigned char* const xsb = xring + frow * 128;
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
      for (int s = 0; s < ns; s += 2) {  // ns is even: every chunk starts in slot 0
        m32_products<TV>(wsb, xsb, fhi, fsw, acc);
        __syncthreads();
        m32_products<TV>(wsb + kMVStage, xsb + kMXStage, fhi, fsw, acc);
        __syncthreads();
      }
      range_epilogue<TV, KEEP>(a, acc, r0 + c * kMV + w4 * (TV * 32), rend, lane & 31, lane >> 5,
                               best);
    }
#pragma unroll
    for (int r = 0; r < kMR; ++r) {
      const uint64_t m = wave_max_u64(best[r]);
      if (lane == 0) wb[w4][r] = m;
    }
    __syncthreads();
  }

  // one publication per request and workgroup: the words of all workgroups
  // meet in eight words of memory, and per-chunk publications by every
  // wave of every CU at nearly the same moment serialise there
  if (threadIdx.x < kMR && (int)threadIdx.x < B) {
    const int r = threadIdx.x;
    publish_slot(a.slots, r, umax64(umax64(wb[0][r], wb[1][r]), umax64(wb[2][r], wb[3][r])));
  }
}

// LM-head from 17 requests on: the activations as register operands.
//
// A workgroup computes 128 vocabulary rows x 32 requests (512 activation
// rows, 16 per request: the 15 positions and a padding row that repeats
// position 14).  Each of its eight waves (two per SIMD) owns 4 requests and
// all 128 rows: 2 x 4 tiles of 32x32x16 products (128 accumulators).  Only
// lm_head goes through LDS (whole-line loads into 64-wide k stages with the
// m32 kernel's chunk swizzle, three stages); each wave reads its activation
// fragments straight from a copy of the block's hiddens laid out in fragment
// order (xfrag_pack_kernel, once per call, so every load instruction reads
// 1 KB of whole lines), through a 4-deep register ring of 32-wide k steps,
// and the lm_head fragments of each 16-wide slice one slice ahead of its
// products.  lm_head is staged through registers rather than by direct
// global->LDS copies: the compiler cannot tell those copies from the
// fragment loads and would wait for every load in flight before each LDS
// read.
//
// Measured (LM-head ms): 8B B = 64 1.143 (line kernel 1.143), B = 32 0.638
// (0.644), 27B-class B = 64 1.436 (1.553); the dispatch range is set at
// lmhead_xfrag_used().  One wave per SIMD with 4 x 4
// tiles (256 accumulators) ran at 1.30 ms at 8B B = 64.  Counters at 8B
// B = 64: the matrix cores are busy 56% of the active cycles (line kernel
// 42%), but the part runs this kernel at ~1.9 GHz against ~2.35 GHz for the
// line kernel (active cycles per microsecond), so the two take the same time.
typedef int v4i __attribute__((ext_vector_type(4)));
// fourth word of a raw buffer resource on gfx9-class parts (32-bit data format)
constexpr int kBufferWord3 = 0x00020000;
constexpr int kXfRq = 32;                      // requests per workgroup
constexpr int kXfV = 128;                      // vocabulary rows per workgroup
constexpr int kXfK = 64;                       // k per LDS stage
constexpr int kXfRing = 3;                     // LDS stages
constexpr int kXfA = 4;                        // register ring of 32-wide k steps
constexpr int kXfTA = 2;                       // activation tiles per wave (8 waves)
constexpr int kXfStage = kXfV * kXfK * 2;      // 16 KB
constexpr size_t kXfLds = (size_t)kXfRing * kXfStage;

// XP: activation tile a (32 rows; group a / 16 holds requests 32 (a / 16) ..,
// row R = 32 (a % 16) + l % 32 is request 32 (a / 16) + R / 16 at position
// min(R % 16, 14)), 16-wide k slice s, lane l, element e at
// ((a nk16 + s) 64 + l) 8 + e with k = 16 s + 8 (l / 32) + e.  Requests past
// B repeat request B - 1 (their results are not stored).
__host__ __device__ inline size_t lmhead_xfrag_bytes(int B, int H) {
  return (size_t)((B + kXfRq - 1) / kXfRq) * 16 * 32 * H * 2;
}

__global__ __launch_bounds__(256) void xfrag_pack_kernel(const bf16_t* __restrict__ X, int B,
                                                         int H, bf16_t* __restrict__ XP,
                                                         size_t pieces) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= pieces) return;
  const int nk16 = H / 16;
  const int l = (int)(t & 63);
  const size_t ts = t >> 6;
  const int s = (int)(ts % nk16);
  const int at = (int)(ts / nk16);
  const int R = (at % 16) * 32 + (l & 31);
  const int req = min((at / 16) * kXfRq + R / 16, B - 1), pos = min(R % 16, DOMINO_T - 1);
  const int k = 16 * s + 8 * (l >> 5);
  *reinterpret_cast<uint4*>(XP + t * 8) =
      *reinterpret_cast<const uint4*>(X + ((size_t)req * DOMINO_T + pos) * H + k);
}

// TA activation tiles (2 TA requests) per wave: 4 (four waves, one per SIMD) or 2 (eight
// waves, two per SIMD, 128 accumulators each)
template <int TA>
__global__ __launch_bounds__(64 * 16 / TA) void lmhead_xf_kernel(FusedArgs a) {
  constexpr int kW = 16 / TA;  // waves
  constexpr int kC = 16 / kW;  // lm_head copy blocks per wave and stage
  const int V = a.V, H = a.H, B = a.B;
  const int nvt = (V + kXfV - 1) / kXfV, ngrp = (B + kXfRq - 1) / kXfRq;
  const int j0 = blockIdx.x, xcd = j0 & 7, local = j0 >> 3;
  const int vt = (local / ngrp) * 8 + xcd, grp = local % ngrp;
  if (vt >= nvt) return;  // uniform per workgroup, before any barrier
  const int v0 = vt * kXfV, b0 = grp * kXfRq;
  extern __shared__ __align__(1024) unsigned char ring[];
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int nk16 = H / 16, nst = H / kXfK, nstep = H / 32;

  // lm_head copies: 16 blocks of 8 rows x 128 B per stage, blocks wave + kW i;
  // lane (rr, pp) fetches logical chunk pp ^ ((r >> 1) & 7) of row rr
  const int rr = lane >> 3, pp = lane & 7;
  uint32_t woff[kC];
#pragma unroll
  for (int i = 0; i < kC; ++i) {
    const int blk = wave + kW * i;
    const int r = (blk & 3) * 8 + rr;
    const int v = min(v0 + blk * 8 + rr, V - 1);
    woff[i] = ((uint32_t)v * (uint32_t)H + (uint32_t)(pp ^ ((r >> 1) & 7)) * 8u) * 2u;
  }
  // Both operands are read through buffer resources: a wave-uniform byte
  // offset in a scalar register plus one per-lane offset, so the loads need
  // no 64-bit address registers.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.W, (short)0, (int)((uint64_t)V * H * 2), kBufferWord3);
  v4i VR[kC];  // this wave's part of one lm_head stage on its way to LDS
  auto load_v = [&](int t) {  // stage t (past the end: the last one again)
    const int kb = min(t, nst - 1) * (kXfK * 2);
#pragma unroll
    for (int i = 0; i < kC; ++i) VR[i] = __builtin_amdgcn_raw_buffer_load_b128(wres, (int)woff[i], kb, 0);
  };
  auto store_v = [&](int t) {  // into slot t % ring
    unsigned char* ws = ring + (t % kXfRing) * kXfStage + lane * 16;
#pragma unroll
    for (int i = 0; i < kC; ++i) *reinterpret_cast<v4i*>(ws + (wave + kW * i) * 1024) = VR[i];
  };
  // this wave's activation tiles: TA of its group's 16, each 2 H bytes per
  // row of 32 (1 KB per 16-wide k slice)
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.XP, (short)0, (int)(lmhead_xfrag_bytes(B, H)), kBufferWord3);
  const int xbase = (grp * 16 + wave * TA) * nk16 * 1024, tstride = nk16 * 1024;
  v8s X[kXfA][TA][2];
  auto issue_x = [&](v8s (&dst)[TA][2], int j) {  // 32-wide k step j (clamped)
    const int jc = min(j, nstep - 1);
#pragma unroll
    for (int ta = 0; ta < TA; ++ta)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        dst[ta][h] = __builtin_bit_cast(
            v8s, __builtin_amdgcn_raw_buffer_load_b128(xres, lane * 16,
                                                       xbase + ta * tstride + (2 * jc + h) * 1024, 0));
  };

  v16f acc[TA][4];
#pragma unroll
  for (int ta = 0; ta < TA; ++ta)
#pragma unroll
    for (int tv = 0; tv < 4; ++tv)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[ta][tv][i] = 0.f;

  const int frow = lane & 31, fhi = lane >> 5, fsw = (frow >> 1) & 7;
  // lm_head fragments of 16-wide slice q (step q / 2, stage q / 4)
  auto read_v = [&](v8s (&fv)[4], int q) {
    const unsigned char* vs = ring + ((q >> 2) % kXfRing) * kXfStage + frow * 128;
    const int cofs = ((2 * (q & 3) + fhi) ^ fsw) * 16;
#pragma unroll
    for (int tv = 0; tv < 4; ++tv) fv[tv] = *reinterpret_cast<const v8s*>(vs + tv * 4096 + cofs);
  };
  // Step j (32-wide k): load the activations of step j + 3; at even j also
  // write lm_head stage j / 2 + 1 (loaded two steps earlier) to LDS and load
  // stage j / 2 + 2; at odd j a barrier makes stage (j + 1) / 2 visible.  A
  // stage is read from the second half of step 2t - 1 (the fragments of each
  // 16-wide slice are read one slice ahead of its products) to step 2t + 1;
  // its slot (three of them) is rewritten at step 2t + 4, after the barrier
  // at step 2t + 3.  The prologue covers steps -3..-1.
  load_v(0);
  store_v(0);
  issue_x(X[0], 0);
  issue_x(X[1], 1);
  load_v(1);  // in the place the loop issues it, so the loop's waits hold from the start
  issue_x(X[2], 2);
  __syncthreads();
  v8s fcur[4];
  read_v(fcur, 0);
  for (int j0s = 0; j0s < nstep; j0s += kXfA) {
#pragma unroll
    for (int d = 0; d < kXfA; ++d) {
      const int j = j0s + d;
      if (d & 1) __syncthreads();
      // the scheduling barriers keep the loads in issue order, so the wait
      // for one group never covers a group issued after it
      __builtin_amdgcn_sched_barrier(0);
      issue_x(X[(d + 3) % kXfA], j + 3);
      __builtin_amdgcn_sched_barrier(0);
      if ((d & 1) == 0) {
        store_v(j / 2 + 1);
        load_v(j / 2 + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v8s fnext[4];
        read_v(fnext, 2 * j + h + 1);
#pragma unroll
        for (int ta = 0; ta < TA; ++ta)
#pragma unroll
          for (int tv = 0; tv < 4; ++tv) acc[ta][tv] = mfma32(X[d][ta][h], fcur[tv], acc[ta][tv]);
#pragma unroll
        for (int tv = 0; tv < 4; ++tv) fcur[tv] = fnext[tv];
      }
    }
  }

  // epilogue: base logits (step-major), pool score keys, first-proposal argmax
  const int vl = lane & 31, hh = lane >> 5;
  const int bw = b0 + wave * 2 * TA;  // this wave's first request
  uint64_t best[2 * TA];
#pragma unroll
  for (int r = 0; r < 2 * TA; ++r) best[r] = 0;
#pragma unroll
  for (int ta = 0; ta < TA; ++ta)
#pragma unroll
    for (int tv = 0; tv < 4; ++tv) {
      const int v = v0 + tv * 32 + vl;
      const bool vok = v < V;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int req = bw + 2 * ta + jj;
        const bool ok = vok && req < B;
        float m = -INFINITY;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int i = jj * 8 + ii;
          const int pos = 8 * ((i >> 2) & 1) + 4 * hh + (i & 3);
          const float y = acc[ta][tv][i];
          if (pos < DOMINO_T) {
            m = fmaxf(m, y);
            if (ok) a.base[((size_t)pos * B + req) * V + v] = y;
          }
        }
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (a.keys && hh == 0 && ok) a.keys[(size_t)req * V + v] = orderable(m);
        const uint64_t k0 = pack_key(acc[ta][tv][jj * 8], (uint32_t)v);  // position 0 on hh == 0
        best[2 * ta + jj] = (hh == 0 && vok) ? umax64(best[2 * ta + jj], k0) : best[2 * ta + jj];
      }
    }
#pragma unroll
  for (int r = 0; r < 2 * TA; ++r) {
    const uint64_t m = wave_max_u64(best[r]);
    if (lane == 0 && bw + r < B) publish_slot(a.slots, bw + r, m);
  }
}

// vocabulary tiles per wave by batch: the 128-row workgroup tile doubles the
// workgroup count where lm_head streaming, not the products, bounds the time
constexpr int kM32SmallBatch = 8;

template <int TV>
constexpr size_t kRangeLds = 2 * ((size_t)M32<TV>::kVStage + kMXStage);  // 64 / 128 KB
// The range kernel's chunk is 4 TV tiles of 32 rows: one tile per consumer
// wave (five chunks of an 8B range of 18-19 tiles) up to 4 requests, three
// from 5 (two chunks: fewer epilogues and activation passes).  8B LM-head us
// on one box, TV = 1 (three register sets) / TV = 3 (two): B = 5 245-256 /
// 250-260, 6 248 / 255, 7 252 / 257-261, 8 255-258 / 253-261: within the
// spread between boxes from 5 requests, so those keep TV = 3.
constexpr int kRangeSmallBatch = 4;
// the stage loops run in pairs of 64-wide k stages
bool lmhead_range_supported(int H) { return H % (2 * kMK) == 0; }

constexpr size_t kLds = (size_t)kStages * kSliceBytes;
// line-copy kernel whenever H is a multiple of its 64-wide stage


}  // namespace

void lmhead_fused_prepare() {
  (void)hipFuncSetAttribute((const void*)lmhead_m32_kernel<2>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)M32<2>::kLds);
  (void)hipFuncSetAttribute((const void*)lmhead_m32_kernel<1>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)M32<1>::kLds);
  (void)hipFuncSetAttribute((const void*)lmhead_range_kernel<1, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRangeLds<1>);
  (void)hipFuncSetAttribute((const void*)lmhead_range_kernel<1, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRangeLds<1>);
  (void)hipFuncSetAttribute((const void*)lmhead_range_kernel<3, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRangeLds<3>);
  (void)hipFuncSetAttribute((const void*)lmhead_range_kernel<3, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRangeLds<3>);
  (void)hipFuncSetAttribute((const void*)lmhead_fused_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  (void)hipFuncSetAttribute((const void*)lmhead_lines_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLinesLds);
  (void)hipFuncSetAttribute((const void*)lmhead_xf_kernel<kXfTA>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kXfLds);
}

size_t lmhead_xfrag_elems(int B, int H) { return lmhead_xfrag_bytes(B, H) / 2; }

// Requests are processed in groups of 32.  One group wins from 17 requests
// on, even part full (8B LM-head ms, this kernel / the m32 or line kernel:
// B = 17 0.569 / 0.607, 20 0.588 / 0.607, 24 0.589 / 0.614, 26 0.607 /
// 0.654, 28 0.605 / -, 32 0.638 / 0.644); with two groups the partial one's
// wasted products cost more than they save unless the waste is at most an
// eighth (B = 56-64; B = 40 1.124 / 0.877, 48 1.12 / 0.94).
constexpr int kXfMinBatch = 17;
bool lmhead_xfrag_used(int B, int H) {
  const int padded = (B + kXfRq - 1) / kXfRq * kXfRq;
  return B >= kXfMinBatch && H % 128 == 0 && (B <= kXfRq || 8 * (padded - B) <= padded);
}

bool lmhead_xfrag_possible(int max_batch, int H) {
  for (int b = kXfMinBatch; b <= max_batch; ++b)
    if (lmhead_xfrag_used(b, H)) return true;
  return false;
}

bool lmhead_fused_supported(int H) { return H % 32 == 0; }

void launch_lmhead_fused(const FusedArgs& a, hipStream_t st) {
  // 32-bit byte offsets of the line copies
  const bool offsets32 = (uint64_t)a.V * a.H * 2 < (1ull << 32) &&
                         (uint64_t)a.B * DOMINO_T * a.H * 2 < (1ull << 32);
  if (a.XP && lmhead_xfrag_used(a.B, a.H) && offsets32) {
    const size_t pieces = lmhead_xfrag_elems(a.B, a.H) / 8;
    DLAUNCH(xfrag_pack_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st,
            (const bf16_t*)a.X, a.B, a.H, (bf16_t*)a.XP, pieces);
    const int nvt = (a.V + kXfV - 1) / kXfV, ngrp = (a.B + kXfRq - 1) / kXfRq;
    DLAUNCH(lmhead_xf_kernel<kXfTA>, dim3(8 * ((nvt + 7) / 8) * ngrp), dim3(64 * 16 / kXfTA), kXfLds,
            st, a);
    return;
  }
  if (a.B <= kM32MaxBatch && a.H % kMK == 0 && offsets32) {
    const int ngrp = (a.B + kMR - 1) / kMR;
    if (a.B <= kMR && lmhead_range_supported(a.H)) {
      const int grid = min((a.V + 31) / 32, cu_count());
      // the logits are kept in the caches when a pool reads them back
      if (a.B <= kRangeSmallBatch) {
        if (a.keys) DLAUNCH((lmhead_range_kernel<1, true>), dim3(grid), dim3(512), kRangeLds<1>, st, a);
        else DLAUNCH((lmhead_range_kernel<1, false>), dim3(grid), dim3(512), kRangeLds<1>, st, a);
      } else {
        if (a.keys) DLAUNCH((lmhead_range_kernel<3, true>), dim3(grid), dim3(512), kRangeLds<3>, st, a);
        else DLAUNCH((lmhead_range_kernel<3, false>), dim3(grid), dim3(512), kRangeLds<3>, st, a);
      }
    } else if (a.B <= kM32SmallBatch) {
      const int nvt = (a.V + M32<1>::kMV - 1) / M32<1>::kMV;
      DLAUNCH(lmhead_m32_kernel<1>, dim3(8 * ((nvt + 7) / 8) * ngrp), dim3(256), M32<1>::kLds, st,
              a);
    } else {
      const int nvt = (a.V + M32<2>::kMV - 1) / M32<2>::kMV;
      DLAUNCH(lmhead_m32_kernel<2>, dim3(8 * ((nvt + 7) / 8) * ngrp), dim3(256), M32<2>::kLds, st,
              a);
    }
    return;
  }
  const int nvt = (a.V + kBN - 1) / kBN, ngrp = (a.B + kBJ - 1) / kBJ;
  const int grid = 8 * ((nvt + 7) / 8) * ngrp;
  if (a.H % kStageK == 0)
    DLAUNCH(lmhead_lines_kernel, dim3(grid), dim3(256), kLinesLds, st, a);
  else
    DLAUNCH(lmhead_fused_kernel, dim3(grid), dim3(256), kLds, st, a);
}
