// gdn_gate kernel: per-(token, head) decay and write strength.
//
// GDN mode (gated delta rule parameterisation, Gated DeltaNet, ICLR 2025):
//   log g = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h]),   beta = sigmoid(b[t,h])
// Delta-off mode (parameter list of flashinfer.mamba.ssd_combined_fwd: dt_bias,
// dt_softplus, dt_limit with inclusive limits):
//   dt' = clamp(softplus(dt + dt_bias) | dt + dt_bias, lo, hi),  log g = dt' * A[h],  beta = dt'
// Elementwise and HBM-bound; outputs are fp32 [T, H] (row stride H).
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

template <typename InT, bool kSSD>
__global__ void __launch_bounds__(256) gate_kernel(int64_t T, int H, const InT* __restrict__ a,
                                                   int64_t a_stride, const InT* __restrict__ b,
                                                   int64_t b_stride, const float* __restrict__ A,
                                                   const float* __restrict__ dt_bias, int softplus_on,
                                                   float lo, float hi, float* __restrict__ log_g,
                                                   float* __restrict__ beta) {
  const int64_t total = T * (int64_t)H;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / H;
    const int h = int(idx - t * H);
    const float x = Elem<InT>::load(a, t * a_stride + h);
    const float bias = dt_bias ? dt_bias[h] : 0.0f;
    float lg, bt;
    if constexpr (kSSD) gate_ssd(x, A[h], bias, softplus_on, lo, hi, lg, bt);
    else gate_gdn(x, Elem<InT>::load(b, t * b_stride + h), expf(A[h]), bias, lg, bt);
    log_g[idx] = lg;
    beta[idx] = bt;
  }
}

hipError_t launch_gate(const GateLaunch& p, hipStream_t stream) {
  const int64_t total = p.T * (int64_t)p.H;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  dim3 grid((unsigned)blocks), block(threads);
#define GATE_LAUNCH(InT, SSD)                                                                     \
  hipLaunchKernelGGL((gate_kernel<InT, SSD>), grid, block, 0, stream, p.T, p.H,                   \
                     (const InT*)p.a, p.a_stride, (const InT*)p.b, p.b_stride, p.A, p.dt_bias,    \
                     p.dt_softplus, p.dt_min, p.dt_max, p.log_g, p.beta)
  if (p.bf16) {
    if (p.ssd) GATE_LAUNCH(u16, true); else GATE_LAUNCH(u16, false);
  } else {
    if (p.ssd) GATE_LAUNCH(float, true); else GATE_LAUNCH(float, false);
  }
#undef GATE_LAUNCH
  return hipGetLastError();
}

}  // namespace gdn
