// Device helpers shared by the rollout kernels (gfx950 / CDNA4, wave64).
//
// Matrix-core conventions used throughout.  A 16x16 output tile is built
// with V_MFMA_F32_16X16X32_BF16 (bf16 weights) or V_MFMA_F32_16X16X4_F32
// (fp32 weights).  For a 32-wide slice of the reduction dimension starting at
// k0, lane l (row = l % 16, q = l / 16) holds the 8 consecutive elements
// k0 + 8q .. k0 + 8q + 7 of its row of the A operand (weight rows) and of
// its column of the B operand (activations).  The accumulator register i of
// lane l holds output row 4q + i, column l % 16.  The fp32 path issues eight
// 16x16x4 products per slice, product i taking element i of every lane, so
// both paths read the same 8-element fragments.
//
// fp32 activations meet bf16 weights as a hi/lo pair of bf16 values
// (x = hi + lo + O(2^-17 |x|)); both halves go through the matrix core and
// accumulate into the same fp32 register, so products are exact and only the
// accumulation is fp32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;
typedef short v8s __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define DOMINO_T 15   // proposals per block (block size 16)
#define DOMINO_S 14   // correction steps

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// round-to-nearest-even; inputs are finite
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Index of the calling wave in its workgroup.  It is the same in every lane;
// reading it through readfirstlane lets the compiler know that, so loops and
// branches derived from it stay scalar instead of becoming exec-masked.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ v4f zero4() { return v4f{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ v4f mfma_bf16(v8s a, v8s b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f32(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 8 bf16 -> one fragment register quad
__device__ __forceinline__ v8s load_frag_bf16(const bf16_t* p) {
  return *reinterpret_cast<const v8s*>(p);
}
__device__ __forceinline__ v8s zero_frag() {
  v8s r = {0, 0, 0, 0, 0, 0, 0, 0};
  return r;
}

struct F8 { float v[8]; };

__device__ __forceinline__ F8 load8_f32(const float* p) {
  F8 r;
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
  return r;
}
__device__ __forceinline__ F8 zero8() {
  F8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.v[i] = 0.f;
  return r;
}

// fp32 x8 -> (hi, lo) bf16 fragments
__device__ __forceinline__ void split_hi_lo(const F8& x, v8s& hi, v8s& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t h = f32_to_bf16(x.v[i]);
    float rest = x.v[i] - bf16_to_f32(h);
    hi[i] = (short)h;
    lo[i] = (short)f32_to_bf16(rest);
  }
}

// ---------------------------------------------------------------- argmax keys
// key = (order-preserving bits of y) << 32 | ~id.  The unsigned maximum of
// keys is the largest y, and among equal y the lowest id.  -0.0 is mapped to
// +0.0 first.  Every real key is > 0, so 0 is the "empty" value.
__device__ __forceinline__ uint32_t orderable(float y) {
  uint32_t u = __float_as_uint(y);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t pack_key(float y, uint32_t id) {
  return ((uint64_t)orderable(y) << 32) | (uint64_t)(~id);
}
__device__ __forceinline__ int32_t key_id(uint64_t k) { return (int32_t)(~(uint32_t)k); }
__device__ __forceinline__ float key_value(uint64_t k) { return from_orderable((uint32_t)(k >> 32)); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = umax64(v, shfl_xor_u64(v, m));
  return v;
}

// Publish a candidate to a device-wide argmax word.  The coherent pre-read
// skips most atomics once a good key is in place; the result is the maximum
// whatever the order of arrival.
__device__ __forceinline__ void publish_max(uint64_t* slot, uint64_t key) {
  if (key == 0) return;
  uint64_t cur = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (key > cur) atomicMax((unsigned long long*)slot, (unsigned long long)key);
}

// An argmax word (one per position and request) is kept as kSlotCopies
// copies, each alone on a 128-byte line: a workgroup publishes to the copy
// of its XCD (workgroups are dealt to the eight XCDs in turn), and readers
// take the largest copy.  Atomics that many workgroups aim at one line
// serialise (about 10 ns apiece); at 8 requests the 1024 waves of a pool
// correction published to the one line holding all eight words, which cost
// more than the correction's loads.  Word w of an array starts at word
// w * kSlotSpan; an unwritten copy is zero.
constexpr int kSlotCopies = 8;
constexpr int kSlotLine = 16;                       // u64 words per 128-byte line
constexpr int kSlotSpan = kSlotCopies * kSlotLine;  // u64 words per argmax word
__device__ __forceinline__ void publish_slot(uint64_t* slots, int w, uint64_t key) {
  const int c = (int)((blockIdx.x + blockIdx.y * gridDim.x) & (kSlotCopies - 1));
  publish_max(slots + (size_t)w * kSlotSpan + c * kSlotLine, key);
}
__device__ __forceinline__ uint64_t read_slot(const uint64_t* slots, int w) {
  uint64_t v[kSlotCopies];
#pragma unroll
  for (int c = 0; c < kSlotCopies; ++c) v[c] = slots[(size_t)w * kSlotSpan + c * kSlotLine];
  uint64_t m = v[0];
#pragma unroll
  for (int c = 1; c < kSlotCopies; ++c) m = m > v[c] ? m : v[c];
  return m;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
