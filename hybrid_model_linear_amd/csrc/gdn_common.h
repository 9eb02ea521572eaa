// Device helpers shared by the GDN kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kWave = 64;

// ------------------------------------------------------------------ element IO
// Inputs stored as bf16 are handled as raw 16-bit patterns: widening is a shift,
// narrowing uses the hardware round-to-nearest-even conversion.
__device__ __forceinline__ float bf16_to_f32(u16 h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(u16, b);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<u16> {
  __device__ static __forceinline__ float load(const u16* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ void store(u16* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ------------------------------------------------------------------ scalar maps
// softplus(x) = log(1 + exp(x)) = max(x, 0) + log1p(exp(-|x|)); no overflow for large x.
__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.0f) + log1pf(__expf(-fabsf(x)));
}
// sigmoid(x) = 1 / (1 + exp(-x)), evaluated on the side that cannot overflow.
__device__ __forceinline__ float sigmoid_f(float x) {
  if (x >= 0.0f) return 1.0f / (1.0f + __expf(-x));
  float e = __expf(x);
  return e / (1.0f + e);
}

// ------------------------------------------------------------------ wave reductions
// Sum over aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace gdn
