// Matrix-core operand fragments shared by the step kernels (see common.h
// for the lane layout): weight rows (A operand) and
// fp32 activations split into a bf16 hi/lo pair.
#pragma once
#include <type_traits>

#include "common.h"

template <bool BF>
using W_t = typename std::conditional<BF, bf16_t, float>::type;

// ---------------------------------------------------------------- fragments
// Weight-side (A operand) fragment: 8 consecutive elements of one row.
template <bool BF>
struct WFrag;
template <>
struct WFrag<true> {
  v8s f;
  __device__ __forceinline__ void load(const bf16_t* p) { f = load_frag_bf16(p); }
};
template <>
struct WFrag<false> {
  F8 f;
  __device__ __forceinline__ void load(const float* p) { f = load8_f32(p); }
};

// Activation fragment of fp32 values (GRU state, projector output).
template <bool BF>
struct HFrag;
template <>
struct HFrag<true> {
  v8s hi, lo;
  __device__ __forceinline__ void load(const float* p, bool ok) {
    if (ok) {
      split_hi_lo(load8_f32(p), hi, lo);
    } else {
      hi = zero_frag();
      lo = zero_frag();
    }
  }
};
template <>
struct HFrag<false> {
  F8 f;
  __device__ __forceinline__ void load(const float* p, bool ok) { f = ok ? load8_f32(p) : zero8(); }
};

__device__ __forceinline__ v4f mma(const WFrag<true>& a, const HFrag<true>& x, v4f c) {
  c = mfma_bf16(a.f, x.hi, c);
  return mfma_bf16(a.f, x.lo, c);
}
__device__ __forceinline__ v4f mma(const WFrag<false>& a, const HFrag<false>& x, v4f c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = mfma_f32(a.f.v[i], x.f.v[i], c);
  return c;
}

template <bool BF>
__device__ __forceinline__ float load_w(const W_t<BF>* p) {
  if constexpr (BF) {
    return bf16_to_f32(*p);
  } else {
    return *p;
  }
}
