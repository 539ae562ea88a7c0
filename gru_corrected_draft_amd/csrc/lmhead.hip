// Base LM-head logits of the whole draft block, full vocabulary:
//   base[t, b, v] = sum_i hidden[b, t, i] * lm_head[v, i]      (fp32 out)
// "Add correctness-first Domino support to DFlash V2" (sglang PR #31328),
// "Design": the base projection stays full-vocabulary and is computed once
// per block; "feat: support tensor-parallel Domino rollout" (sglang PR
// #32018), "Rollout performance": step-major packing.  Activation row
// m = t * B + b is read straight from hidden[b, t, :] (the packing is only an
// index map), so the output rows come out step-major.
//
// Two kernels:
//  * stream (M = 15B <= 128): each wave owns 64 vocabulary rows and streams
//    them from HBM once against all M activation rows (bandwidth-bound);
//  * tiled (bf16, M > 128): 128 x 128 output tiles, 64-deep k-steps staged
//    through LDS with double buffering (matrix-core-bound).  Tiles that share
//    lm_head rows run back to back on one XCD so the rows are fetched into
//    that XCD's L2 once.
#include <type_traits>

#include "common.h"
#include "launch.h"

template <bool BF>
using W_t = typename std::conditional<BF, bf16_t, float>::type;

template <bool BF, int NB>
__global__ __launch_bounds__(256) void lmhead_stream_kernel(const W_t<BF>* __restrict__ W,
                                                            const W_t<BF>* __restrict__ X,
                                                            float* __restrict__ out, int V, int H,
                                                            int B) {
  const int M = B * DOMINO_T;
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;
  const int v0 = (blockIdx.x * 4 + wave) * 64;
  if (v0 >= V) return;  // no workgroup barrier in this kernel
  const W_t<BF>* pw[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) pw[t] = W + (size_t)min(v0 + t * 16 + row, V - 1) * H + q * 8;

  for (int m0 = 0; m0 < M; m0 += NB * 16) {
    const W_t<BF>* px[NB];
    bool xv[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int m = m0 + cb * 16 + row;
      xv[cb] = m < M;
      const int mm = xv[cb] ? m : 0;
      px[cb] = X + ((size_t)(mm % B) * DOMINO_T + mm / B) * H + q * 8;
    }
    v4f acc[4][NB];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) acc[t][cb] = zero4();


    for (int k = 0; k < H; k += 32) {
      if constexpr (BF) {
        v8s a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = load_frag_bf16(pw[t] + k);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const v8s x = xv[cb] ? load_frag_bf16(px[cb] + k) : zero_frag();
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t][cb] = mfma_bf16(a[t], x, acc[t][cb]);
        }
      } else {
        F8 a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = load8_f32(pw[t] + k);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const F8 x = xv[cb] ? load8_f32(px[cb] + k) : zero8();
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[t][cb] = mfma_f32(a[t].v[i], x.v[i], acc[t][cb]);
        }
      }
    }
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int m = m0 + cb * 16 + row;
      if (m >= M) continue;
      float* orow = out + (size_t)m * V;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int v = v0 + t * 16 + 4 * q;
        if ((V & 3) == 0 && v + 3 < V) {
          *reinterpret_cast<float4*>(orow + v) =
              make_float4(acc[t][cb][0], acc[t][cb][1], acc[t][cb][2], acc[t][cb][3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v + i < V) orow[v + i] = acc[t][cb][i];
        }
      }
    }
  }
}

// ----------------------------------------------------------- tiled (bf16)
constexpr int kTV = 128, kTM = 128, kTK = 64, kLdsRow = kTK + 8;  // padded LDS rows

__global__ __launch_bounds__(256) void lmhead_tiled_kernel(const bf16_t* __restrict__ W,
                                                           const bf16_t* __restrict__ X,
                                                           float* __restrict__ out, int V, int H,
                                                           int B, int nvt, int nmt) {
  const int M = B * DOMINO_T;
  // workgroups are dealt to the 8 XCDs round robin: give every XCD whole
  // vocabulary tiles and walk their m tiles consecutively
  const int j = blockIdx.x, xcd = j & 7, local = j >> 3;
  const int vt = (local / nmt) * 8 + xcd, mt = local % nmt;
  if (vt >= nvt) return;  // uniform per workgroup, before any barrier
  const int v0 = vt * kTV, m0 = mt * kTM;

  extern __shared__ __align__(16) bf16_t lds[];
  bf16_t* As = lds;                          // [2][kTV][kLdsRow]
  bf16_t* Bs = lds + 2 * kTV * kLdsRow;      // [2][kTM][kLdsRow]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, q = lane >> 4;
  const int wv = wave & 1, wm = wave >> 1;   // 2 x 2 waves, 64 x 64 each

  // global -> LDS copy map: 1024 16-byte pieces per operand tile
  const bf16_t* ga[4];
  const bf16_t* gb[4];
  bool bok[4];
  int lr[4], lc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int idx = tid + 256 * p;
    lr[p] = idx >> 3;
    lc[p] = (idx & 7) * 8;
    ga[p] = W + (size_t)min(v0 + lr[p], V - 1) * H + lc[p];
    const int m = m0 + lr[p];
    bok[p] = m < M;
    const int mm = bok[p] ? m : 0;
    gb[p] = X + ((size_t)(mm % B) * DOMINO_T + mm / B) * H + lc[p];
  }
  uint4 ra[4], rb[4];
  const uint4 z4 = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    ra[p] = *reinterpret_cast<const uint4*>(ga[p]);
    rb[p] = bok[p] ? *reinterpret_cast<const uint4*>(gb[p]) : z4;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    *reinterpret_cast<uint4*>(&As[lr[p] * kLdsRow + lc[p]]) = ra[p];
    *reinterpret_cast<uint4*>(&Bs[lr[p] * kLdsRow + lc[p]]) = rb[p];
  }
  __syncthreads();

  v4f acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[t][c] = zero4();

  const int nk = H / kTK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k = (kt + 1) * kTK;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        ra[p] = *reinterpret_cast<const uint4*>(ga[p] + k);
        rb[p] = bok[p] ? *reinterpret_cast<const uint4*>(gb[p] + k) : z4;
      }
    }
    const bf16_t* Ac = As + cur * kTV * kLdsRow;
    const bf16_t* Bc = Bs + cur * kTM * kLdsRow;
#pragma unroll
    for (int kc = 0; kc < kTK / 32; ++kc) {
      v8s af[4], bfr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        af[t] = load_frag_bf16(&Ac[(wv * 64 + t * 16 + row) * kLdsRow + kc * 32 + q * 8]);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        bfr[c] = load_frag_bf16(&Bc[(wm * 64 + c * 16 + row) * kLdsRow + kc * 32 + q * 8]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[t][c] = mfma_bf16(af[t], bfr[c], acc[t][c]);
    }
    if (more) {
      bf16_t* An = As + (cur ^ 1) * kTV * kLdsRow;
      bf16_t* Bn = Bs + (cur ^ 1) * kTM * kLdsRow;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        *reinterpret_cast<uint4*>(&An[lr[p] * kLdsRow + lc[p]]) = ra[p];
        *reinterpret_cast<uint4*>(&Bn[lr[p] * kLdsRow + lc[p]]) = rb[p];
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int m = m0 + wm * 64 + c * 16 + row;
    if (m >= M) continue;
    float* orow = out + (size_t)m * V;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int v = v0 + wv * 64 + t * 16 + 4 * q;
      if ((V & 3) == 0 && v + 3 < V) {
        *reinterpret_cast<float4*>(orow + v) =
            make_float4(acc[t][c][0], acc[t][c][1], acc[t][c][2], acc[t][c][3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v + i < V) orow[v + i] = acc[t][c][i];
      }
    }
  }
}

template <bool BF, int NB>
static void stream_launch(const Shape& s, const void* W, const void* X, float* out, int B,
                          hipStream_t st) {
  const int units = (s.V + 63) / 64;
  DLAUNCH((lmhead_stream_kernel<BF, NB>), dim3((units + 3) / 4), dim3(256), 0, st,
                     (const W_t<BF>*)W, (const W_t<BF>*)X, out, s.V, s.H, B);
}

template <bool BF>
static void stream_dispatch(const Shape& s, const void* W, const void* X, float* out, int B,
                            hipStream_t st) {
  const int nb = (B * DOMINO_T + 15) / 16;
  switch (nb < 8 ? nb : 8) {
    case 1: stream_launch<BF, 1>(s, W, X, out, B, st); break;
    case 2: stream_launch<BF, 2>(s, W, X, out, B, st); break;
    case 3: stream_launch<BF, 3>(s, W, X, out, B, st); break;
    case 4: stream_launch<BF, 4>(s, W, X, out, B, st); break;
    case 5: stream_launch<BF, 5>(s, W, X, out, B, st); break;
    case 6: stream_launch<BF, 6>(s, W, X, out, B, st); break;
    case 7: stream_launch<BF, 7>(s, W, X, out, B, st); break;
    default: stream_launch<BF, 8>(s, W, X, out, B, st); break;
  }
}

constexpr size_t kTiledLds = (size_t)2 * (kTV + kTM) * kLdsRow * sizeof(bf16_t);

void lmhead_prepare() {
  (void)hipFuncSetAttribute((const void*)lmhead_tiled_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)kTiledLds);
}

void launch_lmhead(const Shape& s, const void* W, const void* X, float* out, int B,
                   hipStream_t st) {
  const int M = B * DOMINO_T;
  if (!s.bf16) {
    stream_dispatch<false>(s, W, X, out, B, st);
  } else if (M <= 128 && rowstream_supported(s.H, M)) {
    StreamArgs a{(const uint16_t*)W, s.V, s.H, (const uint16_t*)X, nullptr, M, B, 0, out,
                 nullptr, nullptr, nullptr, 0};
    launch_rowstream_store(a, st);
  } else if (M <= 128) {
    stream_dispatch<true>(s, W, X, out, B, st);
  } else {
    const int nvt = (s.V + kTV - 1) / kTV, nmt = (M + kTM - 1) / kTM;
    const int grid = 8 * ((nvt + 7) / 8) * nmt;
    DLAUNCH(lmhead_tiled_kernel, dim3(grid), dim3(256), kTiledLds, st,
                       (const bf16_t*)W, (const bf16_t*)X, out, s.V, s.H, B, nvt, nmt);
  }
}
