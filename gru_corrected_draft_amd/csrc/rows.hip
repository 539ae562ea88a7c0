// Latency-oriented GRU cell and fc1 + SiLU for small batches (bf16 weights).
//
// One wave owns one output unit: the GRU's hidden unit j (its six weight
// rows W_ih[r|z|n][j], W_hh[r|z|n][j]) or the projector's unit i (row
// fc1[i]).  Every lane issues all of its weight loads at once (8-byte
// slices, k = 256*it + 4*lane + 0..3), so a launch has the whole weight
// matrix in flight across ~g waves; the requests are then walked with the
// weights held in registers and each dot product finished by a cross-lane
// reduction.  GRU gate algebra: "Add correctness-first Domino support to
// DFlash V2" (sglang PR #31328), section "Design" (bias-free GRU, PyTorch
// gate order r, z, n).
#include "common.h"
#include "launch.h"

namespace {

__device__ __forceinline__ void load4(const bf16_t* p, float (&w)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  w[0] = __uint_as_float(v.x << 16);
  w[1] = __uint_as_float(v.x & 0xFFFF0000u);
  w[2] = __uint_as_float(v.y << 16);
  w[3] = __uint_as_float(v.y & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const float* p, float (&w)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  w[0] = v.x;
  w[1] = v.y;
  w[2] = v.z;
  w[3] = v.w;
}

// 4 consecutive elements at k of a row of length n (n % 4 == 0), or zeros when
// k >= n.  The address is clamped instead of branched on, so consecutive
// loads issue back to back without a wait between them; a masked lane reads
// the row's first 4 elements, which exist for every row this file reads
// (n may be 0 when the row is not used at all, e.g. W_hh with h = 0).
template <typename T>
__device__ __forceinline__ void load4z(const T* row, int k, int n, float (&w)[4]) {
  const bool ok = k < n;
  load4(row + (ok ? k : 0), w);
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = ok ? w[i] : 0.f;
}

// Sum four per-lane values over the wave.  Afterwards lane l holds the total
// of value ((l >> 5) & 1) * 2 + ((l >> 4) & 1): lanes 0..15 value 0, 16..31
// value 1, 32..47 value 2, 48..63 value 3.
__device__ __forceinline__ float reduce4(float v0, float v1, float v2, float v3) {
  const int l = threadIdx.x & 63;
  const bool h5 = l & 32, h4 = l & 16;
  const float s0 = h5 ? v0 : v2, s1 = h5 ? v1 : v3;
  const float a0 = (h5 ? v2 : v0) + __shfl_xor(s0, 32, 64);
  const float a1 = (h5 ? v3 : v1) + __shfl_xor(s1, 32, 64);
  float b = (h4 ? a1 : a0) + __shfl_xor(h4 ? a0 : a1, 16, 64);
  b += __shfl_xor(b, 8, 64);
  b += __shfl_xor(b, 4, 64);
  b += __shfl_xor(b, 2, 64);
  b += __shfl_xor(b, 1, 64);
  return b;
}

// IE / IG: 256-wide k blocks of the embedding and GRU widths
template <int IE, int IG>
__global__ __launch_bounds__(256) void gru_rows_kernel(GruArgs16 a) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= a.g) return;  // no barrier in this kernel
  const int e = a.e, g = a.g;
  float wi[3][IE][4], wh[3][IG][4];
#pragma unroll
  for (int gt = 0; gt < 3; ++gt) {
#pragma unroll
    for (int it = 0; it < IE; ++it) {
      load4z(a.w_ih + ((size_t)gt * g + j) * e, it * 256 + lane * 4, e, wi[gt][it]);
    }
#pragma unroll
    for (int it = 0; it < IG; ++it) {
      load4z(a.w_hh + ((size_t)gt * g + j) * g, it * 256 + lane * 4, a.h_in ? g : 0, wh[gt][it]);
    }
  }
  // lane l fetches the token of request l once
  int my_tok = 0;
  if (lane < a.B) {
    my_tok = a.tok_key ? key_id(a.tok_key[lane]) : a.tok_i32[(size_t)lane * a.tok_stride];
    if (my_tok < 0 || my_tok >= a.V) {
      if (j == 0) a.bad[lane] = 1;
      my_tok = 0;
    }
  }
  // activations of request b+1 are fetched while request b is reduced
  float x[IE][4], hv[IG][4], xn[IE][4], hn[IG][4];
  auto fetch = [&](int b, float (&xx)[IE][4], float (&hh)[IG][4]) {
    const int tok = __shfl(my_tok, b, 64);
#pragma unroll
    for (int it = 0; it < IE; ++it) {
      load4z(a.E + (size_t)tok * e, it * 256 + lane * 4, e, xx[it]);
    }
#pragma unroll
    for (int it = 0; it < IG; ++it) {
      if (a.h_in) load4z(a.h_in + (size_t)b * g, it * 256 + lane * 4, g, hh[it]);
      else hh[it][0] = hh[it][1] = hh[it][2] = hh[it][3] = 0.f;
    }
  };
  fetch(0, x, hv);
  for (int b = 0; b < a.B; ++b) {
    if (b + 1 < a.B) fetch(b + 1, xn, hn);
    float pr = 0.f, pz = 0.f, an = 0.f, cn = 0.f;
#pragma unroll
    for (int it = 0; it < IE; ++it)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr += wi[0][it][i] * x[it][i];
        pz += wi[1][it][i] * x[it][i];
        an += wi[2][it][i] * x[it][i];
      }
#pragma unroll
    for (int it = 0; it < IG; ++it)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr += wh[0][it][i] * hv[it][i];
        pz += wh[1][it][i] * hv[it][i];
        cn += wh[2][it][i] * hv[it][i];
      }
    const float tot = reduce4(pr, pz, an, cn);
    const float S_r = __shfl(tot, 0, 64), S_z = __shfl(tot, 16, 64);
    const float S_an = __shfl(tot, 32, 64), S_cn = __shfl(tot, 48, 64);
    if (lane == 0) {
      const float hold = a.h_in ? a.h_in[(size_t)b * g + j] : 0.0f;
      const float rg = sigmoidf_(S_r);
      const float zg = sigmoidf_(S_z);
      const float ng = tanhf(S_an + rg * S_cn);
      a.h_out[(size_t)b * g + j] = (1.0f - zg) * ng + zg * hold;
    }
#pragma unroll
    for (int it = 0; it < IE; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) x[it][c] = xn[it][c];
#pragma unroll
    for (int it = 0; it < IG; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) hv[it][c] = hn[it][c];
  }
}

template <int IG>
__global__ __launch_bounds__(256) void fc1_rows_kernel(Fc1Args16 a) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= a.r) return;
  const int g = a.g, r = a.r;
  float w[IG][4];
#pragma unroll
  for (int it = 0; it < IG; ++it) {
    load4z(a.F1 + (size_t)i * g, it * 256 + lane * 4, g, w[it]);
  }
  for (int b0 = 0; b0 < a.B; b0 += 4) {
    float d[4];
    float hv[4][IG][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = min(b0 + u, a.B - 1);  // rows past the batch are computed and dropped
#pragma unroll
      for (int it = 0; it < IG; ++it) load4z(a.h + (size_t)b * g, it * 256 + lane * 4, g, hv[u][it]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      d[u] = 0.f;
#pragma unroll
      for (int it = 0; it < IG; ++it)
#pragma unroll
        for (int c = 0; c < 4; ++c) d[u] += w[it][c] * hv[u][it][c];
    }
    const float z = reduce4(d[0], d[1], d[2], d[3]);
    const int b = b0 + (lane >> 4);
    if ((lane & 15) == 0 && b < a.B) {
      const float v = z + a.s[((size_t)b * DOMINO_S + a.step) * r + i];
      const float uu = v * sigmoidf_(v);
      a.u[(size_t)b * r + i] = uu;
      const uint32_t hi = f32_to_bf16(uu);
      a.u_hi[(size_t)b * r + i] = (uint16_t)hi;
      a.u_lo[(size_t)b * r + i] = (uint16_t)f32_to_bf16(uu - bf16_to_f32(hi));
    }
  }
}

}  // namespace

bool rows_supported(int e, int g, int r) {
  (void)r;
  return (e + 255) / 256 <= 5 && (g + 255) / 256 <= 5 && e % 4 == 0 && g % 4 == 0;
}

void launch_gru_rows(const GruArgs16& a, hipStream_t st) {
  const dim3 grid((a.g + 3) / 4), blk(256);
  const int ie = (a.e + 255) / 256, ig = (a.g + 255) / 256;
#define CASE(E, G)                                                       \
  if (ie == E && ig == G) {                                              \
    DLAUNCH((gru_rows_kernel<E, G>), grid, blk, 0, st, a);    \
    return;                                                              \
  }
  CASE(1, 1) CASE(2, 2) CASE(3, 3) CASE(4, 4) CASE(5, 5)
#undef CASE
  // mixed widths: the largest block count covers both
  const int m = ie > ig ? ie : ig;
  if (m <= 1) DLAUNCH((gru_rows_kernel<1, 1>), grid, blk, 0, st, a);
  else if (m == 2) DLAUNCH((gru_rows_kernel<2, 2>), grid, blk, 0, st, a);
  else if (m == 3) DLAUNCH((gru_rows_kernel<3, 3>), grid, blk, 0, st, a);
  else if (m == 4) DLAUNCH((gru_rows_kernel<4, 4>), grid, blk, 0, st, a);
  else DLAUNCH((gru_rows_kernel<5, 5>), grid, blk, 0, st, a);
}

void launch_fc1_rows(const Fc1Args16& a, hipStream_t st) {
  const dim3 grid((a.r + 3) / 4), blk(256);
  switch ((a.g + 255) / 256) {
    case 1: DLAUNCH((fc1_rows_kernel<1>), grid, blk, 0, st, a); break;
    case 2: DLAUNCH((fc1_rows_kernel<2>), grid, blk, 0, st, a); break;
    case 3: DLAUNCH((fc1_rows_kernel<3>), grid, blk, 0, st, a); break;
    case 4: DLAUNCH((fc1_rows_kernel<4>), grid, blk, 0, st, a); break;
    default: DLAUNCH((fc1_rows_kernel<5>), grid, blk, 0, st, a); break;
  }
}
