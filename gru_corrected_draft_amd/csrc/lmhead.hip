// Base LM-head logits of the whole draft block, full vocabulary:
//   base[t, b, v] = sum_i hidden[b, t, i] * lm_head[v, i]      (fp32 out)
// "Add correctness-first Domino support to DFlash V2" (sglang PR #31328),
// "Design": the base projection stays full-vocabulary and is computed once
// per block; "feat: support tensor-parallel Domino rollout" (sglang PR
// #32018), "Rollout performance": step-major packing.  Activation row
// m = t * B + b is read straight from hidden[b, t, :] (the packing is only an
// index map), so the output rows come out step-major.
//
// This file serves the batches below the fused GEMM (lmhead_fused.hip) and
// the fp32 models: bf16 goes to the row-stream kernel (stream.hip), or, when
// its LDS panel does not fit, to the stream kernel here, in which each wave
// owns 64 vocabulary rows and streams them from HBM once against all M
// activation rows (bandwidth-bound).
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

void launch_lmhead(const Shape& s, const void* W, const void* X, float* out, int B,
                   hipStream_t st) {
  const int M = B * DOMINO_T;
  if (!s.bf16) {
    stream_dispatch<false>(s, W, X, out, B, st);
  } else if (M <= 128 && rowstream_supported(s.H, M)) {
    StreamArgs a{(const uint16_t*)W, s.V, s.H, (const uint16_t*)X, nullptr, M, B, 0, out,
                 nullptr, nullptr, nullptr, 0};
    launch_rowstream_store(a, st);
  } else {
    stream_dispatch<true>(s, W, X, out, B, st);
  }
}
