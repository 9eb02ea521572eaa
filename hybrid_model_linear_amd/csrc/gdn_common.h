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
// sigmoid(x) = 1 / (1 + exp(-x)), evaluated on the side that cannot overflow.
__device__ __forceinline__ float sigmoid_f(float x) {
  if (x >= 0.0f) return 1.0f / (1.0f + __expf(-x));
  float e = __expf(x);
  return e / (1.0f + e);
}

// ------------------------------------------------------------------ gate
// The per-(token, head) decay and write strength, shared by the gate kernel and the
// kernels that fold the gate in (one definition, so both give the same floats).
//   GDN: log g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b)
//   SSD: dt' = clamp(softplus?(dt + dt_bias), lo, hi), log g = dt' * A, beta = dt'
// exp(A_log) is per head and computed once by the caller.  The per-token functions
// are short enough to run inside the layer kernels (a few ulp):
//   exp(x), x <= 0: Cody-Waite reduction x = n ln2 + r, |r| <= ln2 / 2 (ln2 in two
//     parts so that n ln2_hi is exact), then 2^n * 2^(r log2 e) on the hardware exp2;
//   log1p(u), 0 <= u <= 1: 2 atanh(s) with s = u / (2 + u) <= 1/3, the odd series
//     2 s (1 + s^2/3 + s^4/5 + ... + s^14/15) (next term < 2^-25 relative);
//   1 / d: hardware reciprocal plus one Newton step.
__device__ __forceinline__ float gate_exp_nonpos(float x) {
  const float n = rintf(x * 1.4426950408889634f);
  float r = fmaf(-n, 0.693145751953125f, x);
  r = fmaf(-n, 1.428606765330187e-06f, r);
  return ldexpf(__builtin_amdgcn_exp2f(r * 1.4426950408889634f), (int)n);
}
__device__ __forceinline__ float gate_rcp(float d) {
  const float r = __builtin_amdgcn_rcpf(d);
  return fmaf(fmaf(-d, r, 1.0f), r, r);
}
__device__ __forceinline__ float gate_log1p_unit(float u) {
  const float s = u * gate_rcp(2.0f + u);
  const float t = s * s;
  float q = 1.0f / 15.0f;
  q = fmaf(q, t, 1.0f / 13.0f);
  q = fmaf(q, t, 1.0f / 11.0f);
  q = fmaf(q, t, 1.0f / 9.0f);
  q = fmaf(q, t, 1.0f / 7.0f);
  q = fmaf(q, t, 1.0f / 5.0f);
  q = fmaf(q, t, 1.0f / 3.0f);
  q = fmaf(q, t, 1.0f);
  return 2.0f * s * q;
}
// softplus(z) = max(z, 0) + log1p(exp(-|z|)); sigmoid(b) from e = exp(-|b|) on the
// side that cannot overflow.
__device__ __forceinline__ float gate_softplus(float z) {
  return fmaxf(z, 0.0f) + gate_log1p_unit(gate_exp_nonpos(-fabsf(z)));
}
__device__ __forceinline__ float gate_sigmoid(float b) {
  const float e = gate_exp_nonpos(-fabsf(b));
  const float r = gate_rcp(1.0f + e);
  return b >= 0.0f ? r : e * r;
}
__device__ __forceinline__ void gate_gdn(float a, float b, float exp_A_log, float dt_bias, float& log_g,
                                         float& beta) {
  log_g = -exp_A_log * gate_softplus(a + dt_bias);
  beta = gate_sigmoid(b);
}
__device__ __forceinline__ void gate_ssd(float dt, float A, float dt_bias, int softplus_on, float lo,
                                         float hi, float& log_g, float& beta) {
  float x = dt + dt_bias;
  if (softplus_on) x = gate_softplus(x);
  x = fminf(fmaxf(x, lo), hi);
  log_g = x * A;
  beta = x;
}

// ------------------------------------------------------------------ wave reductions
// Sum over aligned groups of W lanes (W a power of two <= 64), in every lane of the
// group; every lane of the wave must be active.  Within a row of 16 lanes by DPP
// moves (swaps within pairs and quads, then the half-row and row mirrors: each step
// adds a lane whose partial sum covers the other half of the span), across rows by
// lane permutes.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "a power of two <= 64");
  if constexpr (W >= 2) v += dpp_row<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  if constexpr (W >= 4) v += dpp_row<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  if constexpr (W >= 8) v += dpp_row<0x141>(v);   // row_half_mirror (lane i <- 7 - i within 8)
  if constexpr (W >= 16) v += dpp_row<0x140>(v);  // row_mirror (lane i <- 15 - i)
  if constexpr (W >= 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (W >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

}  // namespace gdn
