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
#include "common.h"
#include "launch.h"

namespace {

enum { kEpiStore = 0, kEpiArgmax = 1 };

constexpr int kSC = 128;  // k per super-chunk (4 MFMA k-slices of 32)

template <int NB, int RT, bool SPLIT, int EPI>
__global__ __launch_bounds__(256) void rowstream_kernel(StreamArgs a) {
  extern __shared__ __align__(16) bf16_t sact[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, q = lane >> 4;
  const int N = a.N, K = a.K, KS = a.KS, ncols = a.ncols;
  const int ldsrow = KS + 8;  // 16-byte pad per panel row
  const int tile0 = (blockIdx.x * 4 + wave) * RT;
  const bool active = tile0 * 16 < N;

  const bf16_t* pa[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
    pa[t] = a.W + (size_t)min((tile0 + t) * 16 + row, N - 1) * K + q * 8;

  v4f acc[RT][NB];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[t][cb] = zero4();

  v8s A0[RT][4], A1[RT][4];
  auto load_sc = [&](v8s (&A)[RT][4], int k) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) A[t][c] = load_frag_bf16(pa[t] + k + c * 32);
  };
  auto compute_sc = [&](const v8s (&A)[RT][4], int kk) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // columns past the panel read row 0 and are masked to zero afterwards
      v8s bh[NB], bl[NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int col = cb * 16 + row;
        const bf16_t* src = sact + (col < ncols ? col : 0) * ldsrow + kk + c * 32 + q * 8;
        bh[cb] = load_frag_bf16(src);
        if (SPLIT) bl[cb] = load_frag_bf16(src + ncols * ldsrow);
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        if (cb * 16 + row >= ncols) {
          bh[cb] = zero_frag();
          if (SPLIT) bl[cb] = zero_frag();
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t][cb] = mfma_bf16(A[t][c], bh[cb], acc[t][cb]);
        if (SPLIT) {
#pragma unroll
          for (int t = 0; t < RT; ++t) acc[t][cb] = mfma_bf16(A[t][c], bl[cb], acc[t][cb]);
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
    for (int idx = threadIdx.x; idx < ncols * per_row; idx += 256) {
      const int c = idx / per_row, p = idx - c * per_row;
      const int arow = a.col_B ? (c % a.col_B) * DOMINO_T + c / a.col_B : c;
      const size_t g = (size_t)arow * K + slice0 + p * 8;
      *reinterpret_cast<uint4*>(sact + c * ldsrow + p * 8) =
          *reinterpret_cast<const uint4*>(a.act_hi + g);
      if (SPLIT)
        *reinterpret_cast<uint4*>(sact + (ncols + c) * ldsrow + p * 8) =
            *reinterpret_cast<const uint4*>(a.act_lo + g);
    }
    __syncthreads();
  };

  // Super-chunks i = 0 .. nsc-1 in order (k ascending, or descending when
  // a.reverse is set); A0 holds the even ones and A1 the odd ones, each
  // loaded one super-chunk ahead of its use.  A slice is staged whenever the
  // walk enters it.
  const int nsc = K / kSC;
  const bool rev = a.reverse != 0;
  auto chunk = [&](int i) { return rev ? nsc - 1 - i : i; };
  auto enters_slice = [&](int i) {
    const int sc = chunk(i);
    return rev ? (sc % per_slice == per_slice - 1) : (sc % per_slice == 0);
  };
  if (active) load_sc(A0, chunk(0) * kSC);
  for (int i = 0; i < nsc; i += 2) {
    if (enters_slice(i)) stage(chunk(i));
    if (active && i + 1 < nsc) load_sc(A1, chunk(i + 1) * kSC);
    if (active) compute_sc(A0, (chunk(i) % per_slice) * kSC);
    if (i + 1 >= nsc) break;
    if (enters_slice(i + 1)) stage(chunk(i + 1));
    if (active && i + 2 < nsc) load_sc(A0, chunk(i + 2) * kSC);
    if (active) compute_sc(A1, (chunk(i + 1) % per_slice) * kSC);
  }

  if (EPI == kEpiStore) {
    if (!active) return;  // no barrier follows
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int m = cb * 16 + row;
      if (m >= ncols) continue;
      float* orow = a.out + (size_t)m * N;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int v = (tile0 + t) * 16 + 4 * q;
        if ((N & 3) == 0 && v + 3 < N) {
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
      const int b = cb * 16 + row;
      const float* brow = a.base_k + (size_t)(b < ncols ? b : 0) * N;
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
          best[cb] = (active && b < ncols && c < N) ? umax64(best[cb], key) : best[cb];
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
      if (b < ncols)
        publish_max(&a.slot_k[b], umax64(umax64(wb[0][cb][n], wb[1][cb][n]),
                                         umax64(wb[2][cb][n], wb[3][cb][n])));
    }
  }
}

template <int NB, int RT, bool SPLIT, int EPI>
void launch_t(const StreamArgs& a, hipStream_t st) {
  const int tiles = (a.N + 15) / 16;
  const int waves = (tiles + RT - 1) / RT;
  const size_t lds = (size_t)(SPLIT ? 2 : 1) * a.ncols * (a.KS + 8) * sizeof(bf16_t);
  hipLaunchKernelGGL((rowstream_kernel<NB, RT, SPLIT, EPI>), dim3((waves + 3) / 4), dim3(256), lds,
                     st, a);
}

// largest multiple of 128 that divides K with the panel slice within `budget` bytes
int pick_slice(int K, int ncols, int planes, int budget) {
  int best = 128;
  for (int ks = 128; ks <= K; ks += 128)
    if (K % ks == 0 && (size_t)planes * ncols * (ks + 8) * 2 <= (size_t)budget) best = ks;
  return best;
}

template <bool SPLIT, int EPI>
void dispatch(StreamArgs a, hipStream_t st) {
  const int nb = (a.ncols + 15) / 16;
  a.KS = pick_slice(a.K, a.ncols, SPLIT ? 2 : 1, 32 * 1024);
  switch (nb) {
    // one column block of stores: a single row tile per wave streams faster
    case 1: launch_t<1, EPI == kEpiStore ? 1 : 2, SPLIT, EPI>(a, st); break;
    case 2: launch_t<2, 2, SPLIT, EPI>(a, st); break;
    case 3: launch_t<3, 2, SPLIT, EPI>(a, st); break;
    case 4: launch_t<4, 2, SPLIT, EPI>(a, st); break;
    case 5: launch_t<5, 1, SPLIT, EPI>(a, st); break;
    case 6: launch_t<6, 1, SPLIT, EPI>(a, st); break;
    case 7: launch_t<7, 1, SPLIT, EPI>(a, st); break;
    default: launch_t<8, 1, SPLIT, EPI>(a, st); break;
  }
}

}  // namespace

bool rowstream_supported(int K, int ncols) { return K % kSC == 0 && ncols >= 1 && ncols <= 128; }

void launch_rowstream_store(StreamArgs a, hipStream_t st) { dispatch<false, kEpiStore>(a, st); }

void launch_rowstream_argmax(StreamArgs a, hipStream_t st) { dispatch<true, kEpiArgmax>(a, st); }

void rowstream_prepare() {
  // panels up to 64 KB of dynamic LDS
  const int lim = 64 * 1024;
#define SET(NB, RT, SP, EP)                                                                      \
  (void)hipFuncSetAttribute((const void*)rowstream_kernel<NB, RT, SP, EP>,                       \
                            hipFuncAttributeMaxDynamicSharedMemorySize, lim)
  SET(1, 1, false, kEpiStore); SET(2, 2, false, kEpiStore); SET(3, 2, false, kEpiStore);
  SET(4, 2, false, kEpiStore); SET(5, 1, false, kEpiStore); SET(6, 1, false, kEpiStore);
  SET(7, 1, false, kEpiStore); SET(8, 1, false, kEpiStore);
  SET(1, 2, true, kEpiArgmax); SET(2, 2, true, kEpiArgmax); SET(3, 2, true, kEpiArgmax);
  SET(4, 2, true, kEpiArgmax); SET(5, 1, true, kEpiArgmax); SET(6, 1, true, kEpiArgmax);
  SET(7, 1, true, kEpiArgmax); SET(8, 1, true, kEpiArgmax);
#undef SET
}
