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
    publish_max(&a.slots[b0 + tid],
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
    for (int i = 0; i < 4; ++i) dma16(Wb + (aoff[i] + kb), slot + (wave * 4 + i) * 1024);
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

constexpr size_t kLds = (size_t)kStages * kSliceBytes;


}  // namespace

void lmhead_fused_prepare() {
  (void)hipFuncSetAttribute((const void*)lmhead_fused_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
}

bool lmhead_fused_supported(int H) { return H % 32 == 0; }

void launch_lmhead_fused(const FusedArgs& a, hipStream_t st) {
  const int nvt = (a.V + kBN - 1) / kBN, ngrp = (a.B + kBJ - 1) / kBJ;
  const int grid = 8 * ((nvt + 7) / 8) * ngrp;
  DLAUNCH(lmhead_fused_kernel, dim3(grid), dim3(256), kLds, st, a);
}
