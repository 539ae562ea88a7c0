// Streaming matrix-core kernel shared by the LM-head (small batches) and the
// full-vocabulary correction:
//
//     acc[col, row] = sum_k W[row, k] * act[col, k]
//
// for every row of a large bf16 weight matrix W (lm_head or fc2, read from
// HBM exactly once) against a narrow activation panel of at most 128
// columns (draft hiddens, or the projector output u as a hi/lo bf16 pair).
//
// Bandwidth design for gfx950: each wave owns RT tiles of 16 weight rows and
// keeps the next 128-wide k block of its rows in flight (explicit double
// buffer, 16-byte loads, 2*RT*4 loads per lane outstanding) while the matrix
// cores consume the current one; the activation panel sits in LDS in k
// slices, so the only HBM stream is W.  Epilogues: store fp32 logits
// (LM-head) or add base logits + fc2 bias and reduce a packed argmax key per
// request (correction, "[Spec] Add Domino projector support to DFlash
// speculative decoding (V2)", section "Implementation": fused
// SiLU(z+s)·fc2ᵀ + bias + base_logits followed by the argmax).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace {

enum { kEpiStore = 0, kEpiArgmax = 1, kEpiUnion = 2 };
constexpr int kUnionUnitRows = 32;  // rows per unit of the union stream (two 16-row tiles)

constexpr int kSC = 128;  // k per super-chunk (4 MFMA k-slices of 32)
// Padding (bf16 elements) after each activation-panel row in LDS.  With 16
// elements (32 B) the rows of a 1024- or 2048-wide panel start 8 banks apart
// and the 16-byte fragment reads of 16 rows x 4 chunks hit distinct banks; a
// probe of exactly this read pattern counted half of the LDS-active cycles
// as bank conflicts with an 8-element pad and none with 16 (30.5 against
// 32.5 cycles per read at four waves per CU).
constexpr int kPanelPad = 16;
constexpr bool kStraightWalk = true;

// Row spreading (SP, the one-request LM-head).  A 16-row tile T normally
// holds weight rows 16 T .. 16 T + 15; spread, its row r is weight row r S + T
// (S = ceil(N / 16) tiles), so the sixteen rows a wave streams side by side
// are S rows apart instead of adjacent.  A load-only probe on MI355X read
// adjacent 8 KB rows at ~5.3 TB/s and spread ones at ~6.0; in this kernel the
// LM-head at one request went from 251 to 248 us.  (The correction stream,
// 2 KB rows, was slower spread: 49.4 -> 54.1 us, its epilogue then reading
// bias and base values one by one.)
__device__ __forceinline__ int tile_row(bool sp, int T, int r, int S) {
  return sp ? r * S + T : T * 16 + r;
}

template <int NB, int RT, bool SPLIT, int EPI, int D, bool SP = false>
__global__ __launch_bounds__(256) void rowstream_kernel(StreamArgs a) {
  extern __shared__ __align__(16) bf16_t sact[];
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;
  const int N = a.N, K = a.K, KS = a.KS;
  const int ldsrow = KS + kPanelPad;
  // Column groups of NB*16 activation columns: the a.groups blocks that
  // share one set of weight rows are consecutive on one XCD (blocks j and
  // j + 8 land on the same XCD), so all but the first read their tiles from
  // that XCD's L2.
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int grp = local % a.groups;
  const int rowblock = (local / a.groups) * 8 + xcd;
  const int c0 = grp * NB * 16;
  const int ncl = min(NB * 16, a.ncols - c0);  // columns of this block (>= 1)
  const int tile0 = (rowblock * 4 + wave) * RT;
  const bool active = tile0 * 16 < N;
  const int S = (N + 15) / 16;
  static_assert(!SP || EPI == kEpiStore, "spread rows: store epilogue only");

  const bf16_t* pa[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
    pa[t] = a.W + (size_t)min(tile_row(SP, tile0 + t, row, S), N - 1) * K + q * 8;

  v4f acc[RT][NB];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[t][cb] = zero4();

  v8s A[D][RT][4];  // ring of D super-chunks, D - 1 of them in flight
  auto load_sc = [&](v8s (&dst)[RT][4], int k) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[t][c] = load_frag_bf16(pa[t] + k + c * 32);
  };
  auto compute_sc = [&](const v8s (&Ac)[RT][4], int kk) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // columns past the panel read row 0 and are masked to zero afterwards
      v8s bh[NB], bl[NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int col = cb * 16 + row;
        const bf16_t* src = sact + (col < ncl ? col : 0) * ldsrow + kk + c * 32 + q * 8;
        bh[cb] = load_frag_bf16(src);
        if (SPLIT) bl[cb] = load_frag_bf16(src + ncl * ldsrow);
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        if (cb * 16 + row >= ncl) {
          bh[cb] = zero_frag();
          if (SPLIT) bl[cb] = zero_frag();
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t][cb] = mfma_bf16(Ac[t][c], bh[cb], acc[t][cb]);
        if (SPLIT) {
#pragma unroll
          for (int t = 0; t < RT; ++t) acc[t][cb] = mfma_bf16(Ac[t][c], bl[cb], acc[t][cb]);
        }
      }
    }
  };

  // Stage the activation slice that holds super-chunk sc (all threads, so the
  // barriers are uniform; inactive waves only help with the copy).
  const int per_slice = KS / kSC;
  auto stage = [&](int sc) {
    const int slice0 = (sc / per_slice) * KS;
    __syncthreads();  // the previous slice has been consumed
    const int per_row = KS / 8;
    for (int idx = threadIdx.x; idx < ncl * per_row; idx += 256) {
      const int c = idx / per_row, p = idx - c * per_row;
      const int m = c0 + c;
      const int arow = a.col_B ? (m % a.col_B) * DOMINO_T + m / a.col_B : m;
      const size_t g = (size_t)arow * K + slice0 + p * 8;
      *reinterpret_cast<uint4*>(sact + c * ldsrow + p * 8) =
          *reinterpret_cast<const uint4*>(a.act_hi + g);
      if (SPLIT)
        *reinterpret_cast<uint4*>(sact + (ncl + c) * ldsrow + p * 8) =
            *reinterpret_cast<const uint4*>(a.act_lo + g);
    }
    __syncthreads();
  };

  // Super-chunks i = 0 .. nsc-1 in order (k ascending, or descending when
  // a.reverse is set); super-chunk i lives in ring slot i % D and is loaded
  // D - 1 super-chunks ahead of its use.  A slice is staged whenever the walk
  // enters it; the first one before any weight load is issued, so that its
  // barrier does not wait for them.
  const int nsc = K / kSC;
  const bool rev = a.reverse != 0;
  auto chunk = [&](int i) { return rev ? nsc - 1 - i : i; };
  auto enters_slice = [&](int i) {
    const int sc = chunk(i);
    return rev ? (sc % per_slice == per_slice - 1) : (sc % per_slice == 0);
  };
  stage(chunk(0));
  // Loads are unconditional (past the end they repeat the last super-chunk,
  // an L2 hit): a skipped load on one path would make the compiler wait for
  // every outstanding load before each super-chunk.
#pragma unroll
  for (int p = 0; p < D - 1; ++p) load_sc(A[p], chunk(min(p, nsc - 1)) * kSC);
  if (kStraightWalk && per_slice == nsc && nsc % D == 0) {
    // one slice holds all of K: a straight walk, no staging or tail inside
    int i0 = 0;
    do {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        load_sc(A[(d + D - 1) % D], chunk(min(i0 + d + D - 1, nsc - 1)) * kSC);
        compute_sc(A[d], chunk(i0 + d) * kSC);
      }
      i0 += D;
    } while (i0 < nsc);
  } else {
    for (int i0 = 0; i0 < nsc; i0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int i = i0 + d;
        if (i >= nsc) break;
        if (i > 0 && enters_slice(i)) stage(chunk(i));
        load_sc(A[(d + D - 1) % D], chunk(min(i + D - 1, nsc - 1)) * kSC);
        compute_sc(A[d], (chunk(i) % per_slice) * kSC);
      }
    }
  }

  if (EPI == kEpiStore) {
    if (!active) return;  // no barrier follows
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      if (cb * 16 + row >= ncl) continue;
      float* orow = a.out + (size_t)(c0 + cb * 16 + row) * N;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int v = (tile0 + t) * 16 + 4 * q;
        if (SP) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int vs = tile_row(true, tile0 + t, 4 * q + i, S);
            if (vs < N) orow[vs] = acc[t][cb][i];
          }
        } else if ((N & 3) == 0 && v + 3 < N) {
          *reinterpret_cast<float4*>(orow + v) =
              make_float4(acc[t][cb][0], acc[t][cb][1], acc[t][cb][2], acc[t][cb][3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v + i < N) orow[v + i] = acc[t][cb][i];
        }
      }
    }
  } else {
    // every lane loads (clamped addresses) and masks afterwards, so the
    // epilogue's loads are all in flight together
    float bias[RT][4];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bias[t][i] = bf16_to_f32(a.b2[min((tile0 + t) * 16 + 4 * q + i, N - 1)]);
    uint64_t best[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      best[cb] = 0;
      const int b = cb * 16 + row;  // column within the block
      const float* brow = a.base_k + (size_t)(c0 + (b < ncl ? b : 0)) * N;
      float bv[RT][4];
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[t][i] = brow[min((tile0 + t) * 16 + 4 * q + i, N - 1)];
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = (tile0 + t) * 16 + 4 * q + i;
          const float y = bv[t][i] + (acc[t][cb][i] + bias[t][i]);
          const uint64_t key = pack_key(y, (uint32_t)c);
          best[cb] = (active && b < ncl && c < N) ? umax64(best[cb], key) : best[cb];
        }
    }
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
      if (b < ncl)
        publish_slot(a.slot_k, c0 + b, umax64(umax64(wb[0][cb][n], wb[1][cb][n]),
                                         umax64(wb[2][cb][n], wb[3][cb][n])));
    }
  }
}

// Persistent row stream.  Activation columns form groups of NB*16 whose
// panel (SPLIT: hi and lo planes) over all of K stays in LDS for the whole
// launch; every block owns one group and a strided set of row units (RT
// tiles of 16 weight rows), walked as one continuous stream of 128-wide
// super-chunks through a ring of D register buffers, so the weight stream
// never drains between units.  The blocks of all groups that share a row
// unit are consecutive on one XCD and read the unit through its L2.
// Epilogues: store the unit's logits (LM-head), or fold y = base + (W.u + b2)
// into one packed argmax key per request held in registers, published once
// per block at the end (correction).  The union epilogue streams, for each
// group of requests, only the union of their pools (rows taken through the
// group's id list) and folds a (row, request) pair only when the row is in
// that request's pool, with the base value from the members' compact array.  WV waves per block share the panel (8
// when the panel allows one block per CU, so two waves per SIMD overlap
// their products with their loads).
// PK: the weights come from a.Wpk, W repacked in tile order (see
// pack_tiles_kernel): one load instruction of a wave then reads 1 KB of whole
// 128-byte lines instead of sixteen 64-byte pieces of sixteen rows.
template <int NB, int RT, int D, bool VEC, bool SPLIT, int EPI, int WV, bool PK = false>
__global__ __launch_bounds__(WV * 64) void rowpersist_kernel(StreamArgs a) {
  extern __shared__ __align__(16) bf16_t sact[];
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;
  const int K = a.K, G = a.groups;
  const int ldsrow = K + kPanelPad;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int grp = local % G;
  const int N = EPI == kEpiUnion ? a.un[grp] : a.N;  // >= 1
  const int parts = gridDim.x / G;  // the grid is a multiple of 8 * G
  const int part = (local / G) * 8 + xcd;
  const int c0 = grp * a.gcols;
  const int ncl = min(a.gcols, a.ncols - c0);  // 1 .. NB * 16

  // this wave's row units: w, w + stride, ... (walked backwards when reversed)
  const int units = ((N + 15) / 16 + RT - 1) / RT;
  const int w = part * WV + wave, stride = parts * WV;
  int my_n = units > w ? (units - w + stride - 1) / stride : 0;
  if (EPI == kEpiUnion) my_n = min(my_n, a.umaxu);  // the launch sizes umaxu to cover my_n
  const bool rev = a.reverse != 0;
  const int nsc = K / kSC;
  auto unit_of = [&](int j) { return w + (rev ? my_n - 1 - j : j) * stride; };
  auto kchunk = [&](int ci) { return rev ? nsc - 1 - ci : ci; };

  // union: the records of this wave's rows, staged in LDS behind the panel
  // (kUnionUnitRows per unit) so that row ids and epilogue operands are LDS
  // reads, which never wait on the weight stream's loads
  static_assert(EPI != kEpiUnion || RT * 16 == kUnionUnitRows, "union unit rows");
  uint4* srec = nullptr;
  if (EPI == kEpiUnion) {
    srec = reinterpret_cast<uint4*>(sact + 2 * ncl * ldsrow) + (size_t)wave * a.umaxu * kUnionUnitRows;
    const uint4* rec_g = a.urec + (size_t)grp * a.ustride;
    for (int e = lane; e < my_n * kUnionUnitRows; e += 64) {
      const int j = e / kUnionUnitRows, rr = e % kUnionUnitRows;
      srec[e] = rec_g[min(unit_of(j) * kUnionUnitRows + rr, N - 1)];
    }
  }

  {  // the group's panel: hi plane rows [0, ncl), lo plane rows [ncl, 2 ncl)
    const int per_row = K / 8;
    for (int idx = threadIdx.x; idx < ncl * per_row; idx += WV * 64) {
      const int c = idx / per_row, p = idx - c * per_row;
      const int m = c0 + c;
      const int arow = a.col_B ? (m % a.col_B) * DOMINO_T + m / a.col_B : m;
      const size_t g = (size_t)arow * K + p * 8;
      *reinterpret_cast<u32x4*>(sact + c * ldsrow + p * 8) =
          *reinterpret_cast<const u32x4*>(a.act_hi + g);
      if (SPLIT)
        *reinterpret_cast<u32x4*>(sact + (ncl + c) * ldsrow + p * 8) =
            *reinterpret_cast<const u32x4*>(a.act_lo + g);
    }
    __syncthreads();
  }

  // Prefetch cursor (unit pj, chunk pci), D - 1 super-chunks ahead of the
  // consumer.  Past this wave's last unit (or for a wave without units) the
  // rows are clamped into [0, N), so every load stays inside W; such loads
  // are never consumed.  D divides nsc, so super-chunk ci of any unit sits
  // in ring slot ci % D.  prow: the lane's weight row in each tile of the
  // cursor's unit j (union: the staged record's id; a wave without units
  // reads row 0).
  int pj = 0, pci = 0;
  int prow0 = 0, prow1 = 0;
  static_assert(RT <= 2, "row cursor holds two tiles");
  static_assert(!PK || EPI != kEpiUnion, "unions gather rows by id");
  const int ntiles = (N + 15) / 16;
  auto set_rows = [&](int j) {
    if (PK) {  // tile indices, clamped like the rows
      const int u = unit_of(j);
      prow0 = min(max(u * RT, 0), ntiles - 1);
      prow1 = min(max(u * RT + 1, 0), ntiles - 1);
    } else if (EPI == kEpiUnion) {
      const int jj = min(j, my_n - 1);
      prow0 = jj >= 0 ? (int)srec[jj * kUnionUnitRows + row].x : 0;
      prow1 = jj >= 0 ? (int)srec[jj * kUnionUnitRows + 16 + row].x : 0;
    } else {
      const int u = unit_of(j);
      prow0 = min(max((u * RT) * 16 + row, 0), N - 1);
      prow1 = min(max((u * RT + 1) * 16 + row, 0), N - 1);
    }
  };
  set_rows(0);
  v8s A[D][RT][4];
  auto load_next = [&](v8s (&dst)[RT][4]) {
    if (PK) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const bf16_t* p =
            a.Wpk + (((size_t)(t == 0 ? prow0 : prow1) * nsc + kchunk(pci)) * 4 * 64 + lane) * 8;
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[t][c] = load_frag_bf16(p + c * 512);
      }
    } else {
      const int k = kchunk(pci) * kSC + q * 8;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const bf16_t* p = a.W + (size_t)(t == 0 ? prow0 : prow1) * K + k;
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[t][c] = load_frag_bf16(p + c * 32);
      }
    }
    if (++pci == nsc) {
      pci = 0;
      ++pj;
      set_rows(pj);
    }
  };

  v4f acc[RT][NB];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[t][cb] = zero4();
  uint64_t best[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) best[cb] = 0;

  // Loads are unconditional: a load skipped on one path would make the
  // compiler wait for every outstanding load before each super-chunk.
#pragma unroll
  for (int p = 0; p < D - 1; ++p) load_next(A[p]);
  for (int j = 0; j < my_n; ++j) {
    const int u = unit_of(j);
    // argmax epilogue operands of this unit (raw bias bits, widened at use),
    // issued ahead of the unit's remaining weight loads; VEC: N % 4 == 0 and
    // the bias and base rows are 8- and 16-byte aligned, so the 4 rows of a
    // lane come in one load (rows past N are clamped and masked at the fold)
    uint32_t rbias[RT][4];
    float ebase[NB][RT][4];
    uint4 urc[RT][4];  // union: {id, b2 bits, first member slot, member bits} of the lane's rows
    if (EPI == kEpiUnion) {
      const float* mb_g = a.mb_k + (size_t)grp * a.mstride;
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) urc[t][i] = srec[j * kUnionUnitRows + t * 16 + 4 * q + i];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int bl = cb * 16 + row;  // < 32
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t m = urc[t][i].w;
            const bool mem = (m >> bl) & 1u;
            const uint32_t slot = urc[t][i].z + __popc(m & ((1u << bl) - 1u));
            ebase[cb][t][i] = mb_g[mem ? slot : 0u];  // non-members read one shared word
          }
      }
    } else if (EPI == kEpiArgmax && VEC) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int v = min((u * RT + t) * 16 + 4 * q, N - 4);
        const uint2 r2 = *reinterpret_cast<const uint2*>(a.b2 + v);
        rbias[t][0] = r2.x & 0xFFFFu;
        rbias[t][1] = r2.x >> 16;
        rbias[t][2] = r2.y & 0xFFFFu;
        rbias[t][3] = r2.y >> 16;
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int b = cb * 16 + row;
        const float* brow = a.base_k + (size_t)(c0 + (b < ncl ? b : 0)) * N;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int v = min((u * RT + t) * 16 + 4 * q, N - 4);
          // non-temporal: no other block reads these lines, and kept in L2 they
          // would push out fc2 rows the other group's block is about to read
          // (B = 64: 69.5 -> 68.8 us per step)
          const v4f f4 = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(brow + v));
          const float4 f = make_float4(f4[0], f4[1], f4[2], f4[3]);
          ebase[cb][t][0] = f.x;
          ebase[cb][t][1] = f.y;
          ebase[cb][t][2] = f.z;
          ebase[cb][t][3] = f.w;
        }
      }
    } else if (EPI == kEpiArgmax) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) rbias[t][i] = a.b2[min((u * RT + t) * 16 + 4 * q + i, N - 1)];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int b = cb * 16 + row;
        const float* brow = a.base_k + (size_t)(c0 + (b < ncl ? b : 0)) * N;
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ebase[cb][t][i] = __builtin_nontemporal_load(&brow[min((u * RT + t) * 16 + 4 * q + i, N - 1)]);
      }
    }
    int ci0 = 0;  // nsc >= D: at least one pass
    do {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        load_next(A[(d + D - 1) % D]);
        const int kk = kchunk(ci0 + d) * kSC;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v8s bh[NB], bl[NB];
#pragma unroll
          for (int cb = 0; cb < NB; ++cb) {
            const int col = cb * 16 + row;
            const bf16_t* src = sact + (col < ncl ? col : 0) * ldsrow + kk + c * 32 + q * 8;
            bh[cb] = load_frag_bf16(src);
            if (SPLIT) bl[cb] = load_frag_bf16(src + ncl * ldsrow);
            if (col >= ncl) {
              bh[cb] = zero_frag();
              if (SPLIT) bl[cb] = zero_frag();
            }
          }
#pragma unroll
          for (int cb = 0; cb < NB; ++cb) {
#pragma unroll
            for (int t = 0; t < RT; ++t) acc[t][cb] = mfma_bf16(A[d][t][c], bh[cb], acc[t][cb]);
            if (SPLIT) {
#pragma unroll
              for (int t = 0; t < RT; ++t) acc[t][cb] = mfma_bf16(A[d][t][c], bl[cb], acc[t][cb]);
            }
          }
        }
      }
      ci0 += D;
    } while (ci0 < nsc);
    // unit done
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int b = cb * 16 + row;
      if (EPI == kEpiArgmax) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = (u * RT + t) * 16 + 4 * q + i;
            const float y = ebase[cb][t][i] + (acc[t][cb][i] + bf16_to_f32(rbias[t][i]));
            const uint64_t key = pack_key(y, (uint32_t)c);
            best[cb] = (b < ncl && c < N) ? umax64(best[cb], key) : best[cb];
          }
      } else if (EPI == kEpiUnion) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = (u * RT + t) * 16 + 4 * q + i;
            const uint4 rc = urc[t][i];
            const bool mem = c < N && ((rc.w >> b) & 1u);
            const float y = ebase[cb][t][i] + (acc[t][cb][i] + __uint_as_float(rc.y));
            const uint64_t key = pack_key(y, rc.x);
            best[cb] = mem ? umax64(best[cb], key) : best[cb];
          }
      } else if (b < ncl) {
        float* orow = a.out + (size_t)(c0 + b) * N;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int v = (u * RT + t) * 16 + 4 * q;
          if (VEC) {
            if (v < N)
              *reinterpret_cast<float4*>(orow + v) =
                  make_float4(acc[t][cb][0], acc[t][cb][1], acc[t][cb][2], acc[t][cb][3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (v + i < N) orow[v + i] = acc[t][cb][i];
          }
        }
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t][cb] = zero4();
    }
  }
  if (EPI == kEpiStore) return;  // no barrier follows

#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    best[cb] = umax64(best[cb], shfl_xor_u64(best[cb], 16));
    best[cb] = umax64(best[cb], shfl_xor_u64(best[cb], 32));
  }
  __shared__ uint64_t wb[WV][NB][16];
  if (q == 0)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) wb[wave][cb][row] = best[cb];
  __syncthreads();
  if (threadIdx.x < NB * 16) {
    const int cb = threadIdx.x >> 4, n = threadIdx.x & 15;
    const int b = cb * 16 + n;
    uint64_t m = wb[0][cb][n];
#pragma unroll
    for (int v = 1; v < WV; ++v) m = umax64(m, wb[v][cb][n]);
    if (b < ncl) publish_slot(a.slot_k, c0 + b, m);
  }
}

template <int NB, int RT, int D, bool VEC, bool SPLIT, int EPI, int WV, bool PK = false>
void launch_persist_t(const StreamArgs& a, size_t lds, hipStream_t st) {
  static int per_cu = -1;  // resident blocks per CU at this panel size
  static size_t per_cu_lds = 0;
  if (per_cu < 0 || per_cu_lds != lds) {
    per_cu_lds = lds;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, rowpersist_kernel<NB, RT, D, VEC, SPLIT, EPI, WV, PK>, WV * 64, lds) != hipSuccess)
      n = 1;
    per_cu = n < 1 ? 1 : n;
  }
  // a multiple of 8 * groups blocks, about one wave of resident blocks
  const int unit = 8 * a.groups;
  const int want = cu_count() * per_cu;
  const int grid = ((want + unit - 1) / unit) * unit;
  DLAUNCH((rowpersist_kernel<NB, RT, D, VEC, SPLIT, EPI, WV, PK>), dim3(grid), dim3(WV * 64), lds,
          st, a);
}

// panel bytes of one group of `cols` columns over all of K
size_t persist_lds(int K, int cols, bool split) {
  return (size_t)(split ? 2 : 1) * cols * (K + kPanelPad) * sizeof(bf16_t);
}

// gcols: activation columns per group (at most NB * 16)
template <int NB, int RT, int D, bool SPLIT, int EPI, int WV, bool PK = false>
void launch_persist(StreamArgs a, int gcols, hipStream_t st) {
  a.gcols = gcols;
  a.groups = (a.ncols + gcols - 1) / gcols;
  const size_t lds = persist_lds(a.K, min(a.ncols, gcols), SPLIT);
  const bool vec =
      a.N % 4 == 0 && a.N >= 4 &&
      (EPI == kEpiArgmax ? ((reinterpret_cast<uintptr_t>(a.b2) & 7) == 0 &&
                            (reinterpret_cast<uintptr_t>(a.base_k) & 15) == 0)
                         : (reinterpret_cast<uintptr_t>(a.out) & 15) == 0);
  if (vec)
    launch_persist_t<NB, RT, D, true, SPLIT, EPI, WV, PK>(a, lds, st);
  else
    launch_persist_t<NB, RT, D, false, SPLIT, EPI, WV, PK>(a, lds, st);
}

template <int NB, int RT, bool SPLIT, int EPI, int D, bool SP = false>
void launch_t(StreamArgs a, hipStream_t st) {
  const int tiles = (a.N + 15) / 16;
  const int waves = (tiles + RT - 1) / RT;
  const int rowblocks = (waves + 3) / 4;
  const int cols = min(a.ncols, NB * 16);
  a.groups = (a.ncols + NB * 16 - 1) / (NB * 16);
  const size_t lds = (size_t)(SPLIT ? 2 : 1) * cols * (a.KS + kPanelPad) * sizeof(bf16_t);
  DLAUNCH((rowstream_kernel<NB, RT, SPLIT, EPI, D, SP>),
                     dim3(8 * a.groups * ((rowblocks + 7) / 8)), dim3(256), lds, st, a);
}

// largest multiple of 128 that divides K with the panel slice within `budget` bytes
int pick_slice(int K, int ncols, int planes, int budget) {
  int best = 128;
  for (int ks = 128; ks <= K; ks += 128)
    if (K % ks == 0 && (size_t)planes * ncols * (ks + kPanelPad) * 2 <= (size_t)budget) best = ks;
  return best;
}

// Persistent launches keep a group's whole-K panel within this LDS budget
// and need the ring depth to divide the super-chunk count.
constexpr int kPersistBudget = 150 * 1024;
template <int D>
bool persist_fits(int K, int cols, bool split) {
  return (K / kSC) % D == 0 && persist_lds(K, cols, split) <= (size_t)kPersistBudget;
}

// LM-head store: every column in one block, panel slices within
// kStoreBudget.  (A persistent whole-K panel allows one block per CU at
// H = 4096 and streams slower.)
constexpr int kStoreBudget = 32 * 1024;
constexpr int kStoreD = 3;
void dispatch_store(StreamArgs a, hipStream_t st) {
  const int nb = (a.ncols + 15) / 16;
  a.KS = pick_slice(a.K, a.ncols, 1, kStoreBudget);
  switch (nb) {
    // one column block: a single row tile per wave streams faster, its rows spread
    case 1: launch_t<1, 1, false, kEpiStore, kStoreD, true>(a, st); break;
    case 2: launch_t<2, 2, false, kEpiStore, 2>(a, st); break;
    case 3: launch_t<3, 2, false, kEpiStore, 2>(a, st); break;
    case 4: launch_t<4, 2, false, kEpiStore, 2>(a, st); break;
    case 5: launch_t<5, 1, false, kEpiStore, 2>(a, st); break;
    case 6: launch_t<6, 1, false, kEpiStore, 2>(a, st); break;
    case 7: launch_t<7, 1, false, kEpiStore, 2>(a, st); break;
    default: launch_t<8, 1, false, kEpiStore, 2>(a, st); break;
  }
}

// Correction argmax (u as a hi/lo pair): up to 16 requests, and wider
// batches in 32-request groups (132 KB panel at r = 1024), take the
// persistent stream; panels that do not fit run the sliced kernel.
constexpr int kArgmaxRT = 2;
constexpr int kArgmaxD = 2;
constexpr int kArgmaxWV1 = 4;  // waves per block, groups of up to 16 requests
constexpr int kArgmaxWV2 = 8;  // waves per block, 32-request groups (one block per CU)
void dispatch_argmax(StreamArgs a, hipStream_t st) {
  const bool pk = a.Wpk != nullptr;
  if (a.ncols <= 16 && persist_fits<kArgmaxD>(a.K, a.ncols, true)) {
    if (pk)
      launch_persist<1, kArgmaxRT, kArgmaxD, true, kEpiArgmax, kArgmaxWV1, true>(a, a.ncols, st);
    else
      launch_persist<1, kArgmaxRT, kArgmaxD, true, kEpiArgmax, kArgmaxWV1>(a, a.ncols, st);
  } else if (a.ncols <= 16) {
    a.KS = pick_slice(a.K, a.ncols, 2, 32 * 1024);
    launch_t<1, 2, true, kEpiArgmax, 2>(a, st);
  } else if (persist_fits<kArgmaxD>(a.K, 32, true)) {
    if (pk)
      launch_persist<2, kArgmaxRT, kArgmaxD, true, kEpiArgmax, kArgmaxWV2, true>(a, 32, st);
    else
      launch_persist<2, kArgmaxRT, kArgmaxD, true, kEpiArgmax, kArgmaxWV2>(a, 32, st);
  } else {
    a.KS = pick_slice(a.K, min(a.ncols, 64), 2, 32 * 1024);
    launch_t<4, 2, true, kEpiArgmax, 2>(a, st);
  }
}

// Union stream: groups of `group` requests (at most 32), each over its own
// row list of at most `ubound` rows.  Each wave stages the records of its units in LDS
// behind the panel; the count per wave is bounded with the smallest grid the
// launch can choose (one block per CU).
constexpr size_t kUnionLdsLimit = 156 * 1024;
int union_units_per_wave(int groups, int ubound) {
  const int cus = cu_count();
  const int unit = 8 * groups;
  const int parts = ((cus + unit - 1) / unit) * unit / groups;
  const int units = ((ubound + 15) / 16 + kArgmaxRT - 1) / kArgmaxRT;
  const int waves = parts * kArgmaxWV2;
  return max(1, (units + waves - 1) / waves);
}
size_t union_lds(int K, int ncols, int ubound, int group) {
  const int groups = (ncols + group - 1) / group;
  return persist_lds(K, min(ncols, group), true) +
         (size_t)kArgmaxWV2 * union_units_per_wave(groups, ubound) * kUnionUnitRows * sizeof(uint4);
}
void dispatch_union(StreamArgs a, int ubound, int group, hipStream_t st) {
  a.gcols = group;
  a.groups = (a.ncols + group - 1) / group;
  a.umaxu = union_units_per_wave(a.groups, ubound);
  launch_persist_t<2, kArgmaxRT, kArgmaxD, false, true, kEpiUnion, kArgmaxWV2>(
      a, union_lds(a.K, a.ncols, ubound, group), st);
}

// W [N, K] in tile order: for 16-row tile T, super-chunk s (128 k), slice c
// (32 k) and lane l, the 8 elements lane l of a 16x16x32 product reads (row
// 16 T + l % 16, k = 128 s + 32 c + 8 (l / 16)) sit at (((T nsc + s) 4 + c)
// 64 + l) 8.  Rows past N repeat row N - 1 (their results are masked).  One
// thread per 16-byte piece.
__global__ __launch_bounds__(256) void pack_tiles_kernel(const bf16_t* __restrict__ W, int N,
                                                         int K, bf16_t* __restrict__ out,
                                                         size_t pieces) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= pieces) return;
  const int nsc = K / kSC;
  const int l = (int)(t & 63), c = (int)((t >> 6) & 3);
  const size_t ts = t >> 8;
  const int sc = (int)(ts % nsc);
  const size_t T = ts / nsc;
  const size_t R = min(T * 16 + (size_t)(l & 15), (size_t)N - 1);
  const bf16_t* src = W + R * K + sc * kSC + c * 32 + (l >> 4) * 8;
  *reinterpret_cast<uint4*>(out + t * 8) = *reinterpret_cast<const uint4*>(src);
}

}  // namespace

size_t packed_tiles_elems(int N, int K) { return (size_t)(N + 15) / 16 * 16 * K; }

void launch_pack_tiles(const uint16_t* W, int N, int K, uint16_t* out, hipStream_t st) {
  const size_t pieces = packed_tiles_elems(N, K) / 8;
  hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st,
                     (const bf16_t*)W, N, K, (bf16_t*)out, pieces);
}

bool rowstream_supported(int K, int ncols) { return K % kSC == 0 && ncols >= 1 && ncols <= 128; }

bool rowstream_union_supported(int K, int ncols, int ubound, int group) {
  return K % kSC == 0 && (K / kSC) % kArgmaxD == 0 && group >= 1 && group <= kUnionGroup &&
         ncols >= 1 && ncols <= 64 && union_lds(K, ncols, ubound, group) <= kUnionLdsLimit;
}

int rowstream_union_group(int K, int V, int max_batch, int max_k) {
  // the staged records grow with the groups' row lists, the panel with the
  // group: the largest group for which every batch up to max_batch fits
  for (int group : {32, 24, 16}) {
    const int ubound = (int)std::min<long long>(V, (long long)group * max_k);
    bool ok = true;
    for (int n = 1; n <= std::min(max_batch, 64) && ok; ++n)
      ok = rowstream_union_supported(K, n, ubound, group);
    if (ok) return group;
  }
  return 0;
}

void launch_rowstream_union(StreamArgs a, int ubound, int group, hipStream_t st) {
  dispatch_union(a, ubound, group, st);
}

void launch_rowstream_store(StreamArgs a, hipStream_t st) { dispatch_store(a, st); }

void launch_rowstream_argmax(StreamArgs a, hipStream_t st) { dispatch_argmax(a, st); }

void rowstream_prepare() {
  // sliced panels up to 64 KB of dynamic LDS, persistent panels up to the budget
  const int lim = 64 * 1024;
#define SET(NB, RT, SP, EP, D)                                                                   \
  (void)hipFuncSetAttribute((const void*)rowstream_kernel<NB, RT, SP, EP, D>,                    \
                            hipFuncAttributeMaxDynamicSharedMemorySize, lim)
  (void)hipFuncSetAttribute((const void*)rowstream_kernel<1, 1, false, kEpiStore, kStoreD, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, lim);
  SET(2, 2, false, kEpiStore, 2);
  SET(3, 2, false, kEpiStore, 2); SET(4, 2, false, kEpiStore, 2);
  SET(5, 1, false, kEpiStore, 2); SET(6, 1, false, kEpiStore, 2);
  SET(7, 1, false, kEpiStore, 2); SET(8, 1, false, kEpiStore, 2);
  SET(1, 2, true, kEpiArgmax, 2); SET(4, 2, true, kEpiArgmax, 2);
#undef SET
#define SETP(NB, RT, D, VEC, SP, EP, WV, ...)                                                   \
  (void)hipFuncSetAttribute((const void*)rowpersist_kernel<NB, RT, D, VEC, SP, EP, WV, ##__VA_ARGS__>, \
                            hipFuncAttributeMaxDynamicSharedMemorySize, kPersistBudget)
  SETP(1, kArgmaxRT, kArgmaxD, true, true, kEpiArgmax, kArgmaxWV1);
  SETP(1, kArgmaxRT, kArgmaxD, false, true, kEpiArgmax, kArgmaxWV1);
  SETP(2, kArgmaxRT, kArgmaxD, true, true, kEpiArgmax, kArgmaxWV2);
  SETP(2, kArgmaxRT, kArgmaxD, false, true, kEpiArgmax, kArgmaxWV2);
  SETP(1, kArgmaxRT, kArgmaxD, true, true, kEpiArgmax, kArgmaxWV1, true);
  SETP(1, kArgmaxRT, kArgmaxD, false, true, kEpiArgmax, kArgmaxWV1, true);
  SETP(2, kArgmaxRT, kArgmaxD, true, true, kEpiArgmax, kArgmaxWV2, true);
  SETP(2, kArgmaxRT, kArgmaxD, false, true, kEpiArgmax, kArgmaxWV2, true);
  (void)hipFuncSetAttribute(
      (const void*)rowpersist_kernel<2, kArgmaxRT, kArgmaxD, false, true, kEpiUnion, kArgmaxWV2, false>,
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kUnionLdsLimit);
#undef SETP
}
