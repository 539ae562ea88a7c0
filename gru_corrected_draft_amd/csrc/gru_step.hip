// GRU state update and projector layer 1 of the correction steps.
//
// The GRU is the bias-free cell of "Add correctness-first Domino support to
// DFlash V2" (sglang PR #31328), section "Design" (PyTorch gate order r, z, n):
//   a = W_ih x,  c = W_hh h,  r = sigmoid(a_r + c_r),  z = sigmoid(a_z + c_z),
//   n = tanh(a_n + r * c_n),  h' = (1 - z) * n + z * h,
// and projector layer 1 is u = SiLU(fc1 · h + s) ("[Spec] Add Domino projector
// support to DFlash speculative decoding (V2)", section "Implementation").
//
// How the work is arranged on the GPU:
//  * x is always an embedding row E[token], so a = W_ih E[token] is row
//    `token` of the table G = E W_ihᵀ ([V, 3g] fp32) that create() forms once.
//    An update gathers 3g floats of it instead of streaming W_ih.
//  * c = W_hh h needs only the state, so it is computed as soon as the state
//    exists, in the same product as projector layer 1: one pass over the
//    stacked rows [fc1 (r rows); W_hh (3g rows)] multiplied by h.
//  * The gates then need only G[token], c, and the old h, all elementwise.
//
// States: h(1) = GRU(E[verified], 0) and c(1) = W_hh h(1) (prefix); correction
// step k = 1..S computes h(k+1) = GRU(E[p_k], h(k)) from G[p_k], c(k), h(k), then
// u_k = SiLU(fc1 h(k+1) + s[k-1]) and, if another step follows,
// c(k+1) = W_hh h(k+1).
//
// Three arrangements of a step (step_path()):
//  1. step_rows_kernel<GATES = true>: every workgroup evaluates the gates of
//     all requests into LDS (the inputs are a few KB per request and cached),
//     then its waves multiply their stacked rows with h(k+1).  One launch.
//  2. gru_gate_kernel writes h(k+1), then step_rows_kernel<GATES = false>
//     reads it.  Two launches, for batches where repeating the gates in every
//     workgroup costs more than a launch.
//  3. gru_gate_kernel, then step_mfma_kernel: matrix-core products over
//     16-row tiles of the stacked matrix (hi/lo bf16 split of h), optionally
//     split along g over workgroups with a fixed-order combine.
//
// Fragment order (bf16 models, path 3).  A 16x16x32 product reads, in lane l,
// 8 consecutive k of row l % 16 (weights) or of request l % 16 (state),
// starting at 8 (l / 16): sixteen 64-byte pieces of sixteen rows per load.
// Both operands are therefore stored in the order the lanes read them: for
// each 16-row tile (or 16-request block) and 32-wide chunk c of g, 64 lanes x
// 8 bf16 = 1 KB contiguous, so a load covers eight whole 128-byte lines.  The
// weights are packed once at create(); the gate kernel writes the new state
// both as fp32 [B, g] and as this hi/lo pair (two 1 KB planes per chunk).
#include "common.h"
#include "frag.h"
#include "launch.h"

namespace {

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// token of request b from the argmax word or the int32 source; a token
// outside [0, V) flags the request (when `flag`) and reads row 0 instead
__device__ __forceinline__ int step_token(const StepArgs& a, int b, bool flag) {
  int tok = a.tok_key ? key_id(read_slot(a.tok_key, b)) : a.tok_i32[(size_t)b * a.tok_stride];
  if (tok < 0 || tok >= a.V) {
    if (flag) a.bad[b] = 1;
    tok = 0;
  }
  return tok;
}

__device__ __forceinline__ float gate1(float ar, float az, float an, float cr, float cz, float cn,
                                       float hp) {
  const float rg = sigmoidf_(ar + cr);
  const float zg = sigmoidf_(az + cz);
  const float ng = tanhf(an + rg * cn);
  return (1.0f - zg) * ng + zg * hp;
}

// the new state of units j..j+3 of request b (token tok)
__device__ __forceinline__ float4 gates4(const StepArgs& a, int b, int tok, int j) {
  const int g = a.g;
  const float* gr = a.G + (size_t)tok * 3 * g + j;
  const float4 ar = ld4(gr), az = ld4(gr + g), an = ld4(gr + 2 * g);
  float4 cr = make_float4(0.f, 0.f, 0.f, 0.f), cz = cr, cn = cr, hp = cr;
  if (a.h_prev) {
    const float* cp = a.c_prev + (size_t)b * 3 * g + j;
    cr = ld4(cp);
    cz = ld4(cp + g);
    cn = ld4(cp + 2 * g);
    hp = ld4(a.h_prev + (size_t)b * g + j);
  }
  return make_float4(gate1(ar.x, az.x, an.x, cr.x, cz.x, cn.x, hp.x),
                     gate1(ar.y, az.y, an.y, cr.y, cz.y, cn.y, hp.y),
                     gate1(ar.z, az.z, an.z, cr.z, cz.z, cn.z, hp.z),
                     gate1(ar.w, az.w, an.w, cr.w, cz.w, cn.w, hp.w));
}

// result v of stacked row R for request b: projector unit (R < r) or a row
// of W_hh h
template <bool BF>
__device__ __forceinline__ void step_epilogue(const StepArgs& a, int b, int R, float v) {
  const int r = a.r;
  if (R < r) {
    const float x = v + a.s[((size_t)b * DOMINO_S + a.step) * r + R];
    const float uu = x * sigmoidf_(x);
    a.u[(size_t)b * r + R] = uu;
    if (BF) {
      const uint32_t hi = f32_to_bf16(uu);
      a.u_hi[(size_t)b * r + R] = (uint16_t)hi;
      a.u_lo[(size_t)b * r + R] = (uint16_t)f32_to_bf16(uu - bf16_to_f32(hi));
    }
  } else {
    a.c_new[(size_t)b * 3 * a.g + (R - r)] = v;
  }
}

// ------------------------------------------------------------ gates alone
// one thread per 4 units of one request
__global__ __launch_bounds__(256) void gru_gate_kernel(StepArgs a) {
  const int ncol = a.g / 4;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.B * ncol) return;
  const int b = t / ncol, col = t - b * ncol;
  const int tok = step_token(a, b, col == 0);
  const float4 v = gates4(a, b, tok, 4 * col);
  *reinterpret_cast<float4*>(a.h_new + (size_t)b * a.g + 4 * col) = v;
  if (a.hp) {
    // units j..j+3 sit in chunk j / 32, lane (j % 32) / 8 * 16 + b % 16, elements j % 8 ..
    const int j = 4 * col, c = j >> 5, l = ((j & 31) >> 3) * 16 + (b & 15), e = j & 7;
    const size_t o = ((((size_t)(b >> 4) * (a.g >> 5) + c) * 2) * 64 + l) * 8 + e;
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = f32_to_bf16(x[i]);
      lo[i] = f32_to_bf16(x[i] - bf16_to_f32(hi[i]));
    }
    *reinterpret_cast<uint2*>(a.hp + o) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
    *reinterpret_cast<uint2*>(a.hp + o + 512) =
        make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
  }
}

// stacked [fc1; W_hh] rows into fragment order, one thread per (tile, chunk, lane)
__global__ __launch_bounds__(256) void pack_step_weights_kernel(const bf16_t* __restrict__ F1,
                                                                const bf16_t* __restrict__ W_hh,
                                                                bf16_t* __restrict__ Wp, int r,
                                                                int g, int n) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int nch = g >> 5;
  const int l = t & 63, tc = t >> 6;
  const int T = tc / nch, c = tc - T * nch;
  const int R = T * 16 + (l & 15), k = c * 32 + (l >> 4) * 8;
  const bf16_t* src = R < r ? F1 + (size_t)R * g + k : W_hh + (size_t)(R - r) * g + k;
  *reinterpret_cast<uint4*>(Wp + (size_t)t * 8) = *reinterpret_cast<const uint4*>(src);
}

// ------------------------------------------------------------ row kernel
// Sum four per-lane values over the wave.  Afterwards lanes 0..15 hold the
// total of v0, 16..31 of v1, 32..47 of v2 and 48..63 of v3.
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

constexpr int kRowsPerWave = 4;
constexpr int kRowsPerGroup = 4 * kRowsPerWave;  // four waves

// the epilogue of a projector row with its offset s already at hand
template <bool BF>
__device__ __forceinline__ void step_epilogue_s(const StepArgs& a, int b, int R, float v, float sv) {
  if (R < a.r) {
    const int r = a.r;
    const float x = v + sv;
    const float uu = x * sigmoidf_(x);
    a.u[(size_t)b * r + R] = uu;
    if (BF) {
      const uint32_t hi = f32_to_bf16(uu);
      a.u_hi[(size_t)b * r + R] = (uint16_t)hi;
      a.u_lo[(size_t)b * r + R] = (uint16_t)f32_to_bf16(uu - bf16_to_f32(hi));
    }
  } else {
    a.c_new[(size_t)b * 3 * a.g + (R - a.r)] = v;
  }
}

// bf16 weights, NBR >= B requests.  Wave w of workgroup x owns stacked rows
// row0 + 16x + 4w .. +3 (all of one matrix, since r % 16 == 0); lane l holds
// elements k = 256 it + 4 l + 0..3 of each, it < IG.  The weight loads, the
// tokens and the projector offsets of the group's rows are all issued before
// the state is formed, so they are in flight during it.  LDS holds the new
// state of all requests, [B][g] fp32.  Loops over requests are unrolled to
// NBR with clamped indices, so per-request values stay in registers.
template <int IG, int NBR, bool GATES>
__global__ __launch_bounds__(256) void step_rows_kernel(StepArgs a) {
  extern __shared__ float4 hs4[];
  float* hs = reinterpret_cast<float*>(hs4);
  __shared__ float ssh[NBR][kRowsPerGroup];
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int g = a.g, r = a.r, B = a.B;
  const int Rg = a.row0 + blockIdx.x * kRowsPerGroup;
  const int R0 = Rg + wave * kRowsPerWave;
  const bf16_t* wrow = R0 < r ? (const bf16_t*)a.F1 + (size_t)R0 * g
                              : (const bf16_t*)a.W_hh + (size_t)(R0 - r) * g;
  // Issue order: the weights, then the tokens (uniform scalar loads, which
  // drain on their own counter, so they do not wait for the weights), the
  // projector offsets and the gate inputs.  Vector loads drain in order: a
  // vector load waited on before the gates would hold them until every
  // weight had landed, so the offsets go to LDS only just before the barrier.
  // The weights are loaded non-temporally: the correction between two steps
  // then keeps more of its own rows in the caches (8B, one request, K = 2048:
  // block 0.3633 -> 0.3580 ms; at K0 and with 8 requests no change; the
  // matrix-core product for 3 and more requests is slower with them, 8.7 ->
  // 9.7 us at 64 requests, and keeps cached loads).
  uint2 w[kRowsPerWave][IG];
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q)
#pragma unroll
    for (int it = 0; it < IG; ++it) {
      const int k = it * 256 + lane * 4;
      // a lane past the row's end reads the row's first elements and is zeroed below
      const u32x2 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2*>(wrow + (size_t)q * g + (k < g ? k : 0)));
      w[q][it] = make_uint2(v[0], v[1]);
    }
  __builtin_amdgcn_sched_barrier(0);
  int toks[NBR];
  if (GATES) {
#pragma unroll
    for (int b = 0; b < NBR; ++b)
      toks[b] = step_token(a, min(b, B - 1), blockIdx.x == 0 && threadIdx.x == 0 && b < B);
  }
  float sv = 0.f;
  const bool s_lane = Rg < r && threadIdx.x < NBR * kRowsPerGroup;
  if (s_lane) {
    const int b = threadIdx.x / kRowsPerGroup, rr = threadIdx.x % kRowsPerGroup;
    sv = a.s[((size_t)min(b, B - 1) * DOMINO_S + a.step) * r + Rg + rr];
  }

  const int ncol = g / 4;
  if (GATES) {
    for (int col = threadIdx.x; col < ncol; col += 256) {
      float4 v[NBR];
#pragma unroll
      for (int b = 0; b < NBR; ++b) v[b] = gates4(a, min(b, B - 1), toks[b], 4 * col);
      // the state goes to memory once: column c is written by workgroup c % grid
      const bool mine = (int)(col % gridDim.x) == (int)blockIdx.x;
#pragma unroll
      for (int b = 0; b < NBR; ++b) {
        if (b < B) {
          *reinterpret_cast<float4*>(hs + (size_t)b * g + 4 * col) = v[b];
          if (mine) *reinterpret_cast<float4*>(a.h_new + (size_t)b * g + 4 * col) = v[b];
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < B * ncol; i += 256)
      reinterpret_cast<float4*>(hs)[i] = ld4(a.h_new + (size_t)i * 4);
  }
  if (s_lane) ssh[threadIdx.x / kRowsPerGroup][threadIdx.x % kRowsPerGroup] = sv;
  __syncthreads();

  float wf[kRowsPerWave][IG][4];
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q)
#pragma unroll
    for (int it = 0; it < IG; ++it) {
      const bool ok = it * 256 + lane * 4 < g;
      const uint2 v = w[q][it];
      wf[q][it][0] = ok ? __uint_as_float(v.x << 16) : 0.f;
      wf[q][it][1] = ok ? __uint_as_float(v.x & 0xFFFF0000u) : 0.f;
      wf[q][it][2] = ok ? __uint_as_float(v.y << 16) : 0.f;
      wf[q][it][3] = ok ? __uint_as_float(v.y & 0xFFFF0000u) : 0.f;
    }
  const int qr = lane >> 4;  // the row this lane finishes
#pragma unroll
  for (int b = 0; b < NBR; ++b) {
    if (b < B) {
      float d[kRowsPerWave] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int it = 0; it < IG; ++it) {
        const int k = it * 256 + lane * 4;
        const float4 hv = *reinterpret_cast<const float4*>(hs + (size_t)b * g + (k < g ? k : 0));
#pragma unroll
        for (int q = 0; q < kRowsPerWave; ++q)
          d[q] += wf[q][it][0] * hv.x + wf[q][it][1] * hv.y + wf[q][it][2] * hv.z +
                  wf[q][it][3] * hv.w;
      }
      const float tot = reduce4(d[0], d[1], d[2], d[3]);
      if ((lane & 15) == 0)
        step_epilogue_s<true>(a, b, R0 + qr, tot, ssh[b][wave * kRowsPerWave + qr]);
    }
  }
}

// ------------------------------------------------------------ matrix-core kernel
// One workgroup per 16 stacked rows and all B requests (NB blocks of 16).  Its
// eight waves take the 32-wide chunks of g round robin, CPW chunks per pass,
// with every load of a pass (weight fragments and the hi/lo-split state of
// all requests) issued before its first product; the waves' tiles meet in LDS
// in a fixed order.  With gridDim.y > 1 (only for g > 2048) the chunks are
// also split over workgroups, which write partial tiles
// [tile][split][64 requests][16 rows] for step_combine_kernel.
constexpr int kPartTile = 64 * 16;
constexpr int kMfmaWaves = 8;

// state fragment of one request, read from a valid row and zeroed unless ok
__device__ __forceinline__ void load_h(HFrag<true>& f, const float* p, bool ok) {
  F8 x = load8_f32(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x.v[i] = ok ? x.v[i] : 0.f;
  split_hi_lo(x, f.hi, f.lo);
}
__device__ __forceinline__ void load_h(HFrag<false>& f, const float* p, bool ok) {
  f.f = load8_f32(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) f.f.v[i] = ok ? f.f.v[i] : 0.f;
}

template <bool BF, int NB, int CPW>
__global__ __launch_bounds__(512) void step_mfma_kernel(StepArgs a) {
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int row = lane & 15, q = lane >> 4;
  const int R0 = a.row0 + blockIdx.x * 16;
  const int g = a.g, r = a.r, nch = g / 32;
  // bf16: packed operands, chunk c of tile T at ((T nch + c) 64 + lane) 8; fp32: row-major
  const W_t<BF>* pw = BF ? (const W_t<BF>*)a.Wp + ((size_t)(R0 >> 4) * nch * 64 + lane) * 8
                         : (R0 < r ? (const W_t<BF>*)a.F1 + (size_t)(R0 + row) * g
                                   : (const W_t<BF>*)a.W_hh + (size_t)(R0 - r + row) * g) +
                               q * 8;
  const int wstep = BF ? 64 * 8 : 32;  // elements from one chunk to the next
  const float* hrow[NB];
  const bf16_t* hpk[NB];
  bool bok[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int b = cb * 16 + row;
    bok[cb] = b < a.B;
    hrow[cb] = a.h_new + (size_t)min(b, a.B - 1) * g + q * 8;
    hpk[cb] = BF ? a.hp + ((size_t)cb * nch * 2 * 64 + lane) * 8 : nullptr;
  }
  v4f acc[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) acc[cb] = zero4();
  const int stride = kMfmaWaves * gridDim.y;  // chunks between a wave's consecutive chunks
  for (int c0 = blockIdx.y * kMfmaWaves + wave; c0 < nch; c0 += CPW * stride) {
    WFrag<BF> A[CPW];
    HFrag<BF> X[CPW][NB];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = c0 + i * stride;
      const bool live = c < nch;
      const int cc = live ? c : c0;
      A[i].load(pw + (size_t)cc * wstep);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        if constexpr (BF) {
          const bf16_t* p = hpk[cb] + (size_t)cc * 2 * 512;
          const v8s hi = load_frag_bf16(p), lo = load_frag_bf16(p + 512);
          const bool ok = bok[cb] && live;
          X[i][cb].hi = ok ? hi : zero_frag();
          X[i][cb].lo = ok ? lo : zero_frag();
        } else {
          load_h(X[i][cb], hrow[cb] + cc * 32, bok[cb] && live);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      if (c0 + i * stride < nch) {
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[cb] = mma(A[i], X[i][cb], acc[cb]);
      }
    }
  }
  __shared__ float red[kMfmaWaves][NB][256];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][cb][i * 64 + lane] = acc[cb][i];
  __syncthreads();
  if (threadIdx.x >= 256) return;
  // thread t finishes accumulator i = t / 64 of lane l = t % 64: row 4 (l / 16) + i, request l % 16
  const int l = threadIdx.x & 63, i = threadIdx.x >> 6;
  const int rr = 4 * (l >> 4) + i;
  float Z[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    float z = red[0][cb][threadIdx.x];
#pragma unroll
    for (int wv = 1; wv < kMfmaWaves; ++wv) z += red[wv][cb][threadIdx.x];
    Z[cb] = z;
  }
  if (gridDim.y > 1) {
    float* mine = a.partial + ((size_t)blockIdx.x * gridDim.y + blockIdx.y) * kPartTile;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) mine[(cb * 16 + (l & 15)) * 16 + rr] = Z[cb];
    return;
  }
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int b = cb * 16 + (l & 15);
    if (b < a.B) step_epilogue<BF>(a, b, R0 + rr, Z[cb]);
  }
}

// the split partials of every (request, row) in split order; one thread each
template <bool BF>
__global__ __launch_bounds__(256) void step_combine_kernel(StepArgs a, int nsplit) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.B * a.nrows) return;
  const int b = t / a.nrows, rr = t - b * a.nrows;
  const float* p = a.partial + (size_t)(rr >> 4) * nsplit * kPartTile + b * 16 + (rr & 15);
  float z = p[0];
  for (int sp = 1; sp < nsplit; ++sp) z += p[(size_t)sp * kPartTile];
  step_epilogue<BF>(a, b, a.row0 + rr, z);
}

// workgroups per 16-row tile along g: one up to g = 2048 (at most 8 chunks
// per wave), then enough to keep a wave at 8 chunks, at most kStepMaxSplit
int mfma_splits(int g) {
  const int nch = g / 32;
  int ns = 1;
  while (ns < kStepMaxSplit && nch > kMfmaWaves * 8 * ns) ns *= 2;
  return ns;
}

template <bool BF, int NB, int CPW>
void mfma_launch(const StepArgs& a, int ns, hipStream_t st) {
  DLAUNCH((step_mfma_kernel<BF, NB, CPW>), dim3(a.nrows / 16, ns), dim3(512), 0, st, a);
  if (ns > 1)
    DLAUNCH((step_combine_kernel<BF>), dim3((a.B * a.nrows + 255) / 256), dim3(256), 0, st, a,
            ns);
}

template <bool BF, int NB>
void mfma_cpw(const StepArgs& a, hipStream_t st) {
  const int ns = mfma_splits(a.g);
  const int per = (a.g / 32 + kMfmaWaves * ns - 1) / (kMfmaWaves * ns);  // chunks per wave
  if (per <= 1) mfma_launch<BF, NB, 1>(a, ns, st);
  else if (per <= 2) mfma_launch<BF, NB, 2>(a, ns, st);
  else if (per <= 4) mfma_launch<BF, NB, 4>(a, ns, st);
  else if constexpr (NB >= 3) mfma_launch<BF, NB, 5>(a, ns, st);  // 8 would spill registers
  else if (per <= 5) mfma_launch<BF, NB, 5>(a, ns, st);
  else mfma_launch<BF, NB, 8>(a, ns, st);
}

template <bool BF>
void mfma_dispatch(const StepArgs& a, hipStream_t st) {
  switch ((a.B + 15) / 16) {
    case 1: mfma_cpw<BF, 1>(a, st); break;
    case 2: mfma_cpw<BF, 2>(a, st); break;
    case 3: mfma_cpw<BF, 3>(a, st); break;
    default: mfma_cpw<BF, 4>(a, st); break;
  }
}

template <int NBR, bool GATES>
void rows_ig(const StepArgs& a, hipStream_t st) {
  const dim3 grid(a.nrows / kRowsPerGroup), blk(256);
  const size_t lds = (size_t)a.B * a.g * sizeof(float);
  switch ((a.g + 255) / 256) {
    case 1: DLAUNCH((step_rows_kernel<1, NBR, GATES>), grid, blk, lds, st, a); break;
    case 2: DLAUNCH((step_rows_kernel<2, NBR, GATES>), grid, blk, lds, st, a); break;
    case 3: DLAUNCH((step_rows_kernel<3, NBR, GATES>), grid, blk, lds, st, a); break;
    case 4: DLAUNCH((step_rows_kernel<4, NBR, GATES>), grid, blk, lds, st, a); break;
    default: DLAUNCH((step_rows_kernel<5, NBR, GATES>), grid, blk, lds, st, a); break;
  }
}

template <bool GATES>
void rows_dispatch(const StepArgs& a, hipStream_t st) {
  if (a.B <= 1) rows_ig<1, GATES>(a, st);
  else if (a.B <= 2) rows_ig<2, GATES>(a, st);
  else if (a.B <= 4) rows_ig<4, GATES>(a, st);
  else if (a.B <= 8 || GATES) rows_ig<8, GATES>(a, st);
  else rows_ig<16, false>(a, st);
}

}  // namespace

size_t step_partial_floats(int g, int r) {
  const int nrows = r + 3 * g;
  return (size_t)(nrows / 16) * mfma_splits(g) * kPartTile;
}

int step_path(const Shape& s, int B, int forced) {
  const bool rows_ok = s.bf16 && s.g % 4 == 0 && s.g <= 5 * 256 && B <= kStepRowsMaxBatch;
  if (forced == kStepFused) return rows_ok && B <= kStepFusedMaxBatch ? forced : kStepMfma;
  if (forced == kStepRows) return rows_ok ? forced : kStepMfma;
  if (forced == kStepMfma) return kStepMfma;
  if (!rows_ok) return kStepMfma;
  if (B <= kStepFusedAutoMaxBatch) return kStepFused;
  if (B <= kStepRowsAutoMaxBatch) return kStepRows;
  return kStepMfma;
}

size_t step_packed_weight_elems(int g, int r) { return (size_t)(r + 3 * g) * g; }

void launch_pack_step_weights(const Shape& s, const DeviceWeights& w, uint16_t* Wp, hipStream_t st) {
  const int n = (s.r + 3 * s.g) / 16 * (s.g / 32) * 64;
  hipLaunchKernelGGL(pack_step_weights_kernel, dim3((n + 255) / 256), dim3(256), 0, st,
                     (const bf16_t*)w.fc1, (const bf16_t*)w.w_hh, (bf16_t*)Wp, s.r, s.g, n);
}

void launch_gru_gates(const StepArgs& a, hipStream_t st) {
  const int n = a.B * (a.g / 4);
  DLAUNCH(gru_gate_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a);
}

void launch_step_product(const Shape& s, const StepArgs& a, int path, hipStream_t st) {
  if (a.nrows <= 0) return;
  if (path == kStepFused) {
    rows_dispatch<true>(a, st);
  } else if (path == kStepRows) {
    rows_dispatch<false>(a, st);
  } else if (s.bf16) {
    mfma_dispatch<true>(a, st);
  } else {
    mfma_dispatch<false>(a, st);
  }
}

void step_prepare() {
  // the row kernels keep [B][g] fp32 states in LDS: up to 16 requests x 1280 units
  const int lim = kStepRowsMaxBatch * 5 * 256 * (int)sizeof(float);
#define SET1(IG, NBR, GT)                                                                        \
  (void)hipFuncSetAttribute((const void*)step_rows_kernel<IG, NBR, GT>,                         \
                            hipFuncAttributeMaxDynamicSharedMemorySize, lim)
#define SET(IG)                                                                                  \
  SET1(IG, 1, true); SET1(IG, 2, true); SET1(IG, 4, true); SET1(IG, 8, true);                   \
  SET1(IG, 1, false); SET1(IG, 2, false); SET1(IG, 4, false); SET1(IG, 8, false);               \
  SET1(IG, 16, false)
  SET(1);
  SET(2);
  SET(3);
  SET(4);
  SET(5);
#undef SET
#undef SET1
}
