// Measurement helpers (not part of the layer): the achievable HBM copy bandwidth and
// bf16 MFMA rate of the running GPU, so that the layer's kernels can be reported
// against the box's measured peaks as well as the published ones.
#include "gdn_common.h"
#include "gdn_launch.h"
#include "tile_ops.h"

#include <algorithm>

namespace gdn {

namespace {

// dst[i] = src[i] over n 16-byte elements: each workgroup copies whole tiles of 256 x 2
// elements, a thread's two loads (non-temporal: each byte is read once) in flight
// together, coalesced across the wave; the last partial tile element by element.
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
constexpr int kCopyPer = 2;
// src and dst may be the same buffer (in place: every element read and rewritten, as a
// state update does), so they are not declared restrict.
__global__ void __launch_bounds__(256) copy_probe_kernel(const u32x4v* src, u32x4v* dst, int64_t n) {
  const int64_t tile = 256 * kCopyPer;
  const int64_t full = n / tile;
  for (int64_t t = blockIdx.x; t < full; t += gridDim.x) {
    const int64_t b = t * tile + threadIdx.x;
    u32x4v v[kCopyPer];
#pragma unroll
    for (int e = 0; e < kCopyPer; ++e) v[e] = __builtin_nontemporal_load(src + b + 256 * e);
#pragma unroll
    for (int e = 0; e < kCopyPer; ++e) dst[b + 256 * e] = v[e];
  }
  for (int64_t i = full * tile + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

// Four independent chains of 32x32x16 bf16 MFMAs per wave, iters deep; each thread
// writes the sum of its accumulators (so that nothing is optimised away).  Operands
// are small powers of two derived from the lane id: every partial sum stays exact.
__global__ void __launch_bounds__(256) mfma_probe_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  const uint32_t wa = 0x3a803a80u + (uint32_t)(lane & 1), wb = 0x3a803a80u;   // ~2^-10
  a = __builtin_bit_cast(bf16x8, make_uint4(wa, wa, wa, wa));
  b = __builtin_bit_cast(bf16x8, make_uint4(wb, wb, wb, wb));
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  const int64_t n = bytes / 16, tiles = n / (256 * kCopyPer);
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(tiles, 65536));
  hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4v*>(src),
                     static_cast<u32x4v*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace gdn
