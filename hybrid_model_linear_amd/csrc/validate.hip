// gdn_validate_slots: opt-in device-side check of a slot vector (range and
// uniqueness of the non-negative entries); the hot-path kernels trust slots.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

__global__ void clear_flag_kernel(int32_t* flag) { *flag = 0; }

__global__ void __launch_bounds__(256) validate_slots_kernel(const int32_t* __restrict__ slot, int n,
                                                             int64_t num_slots, int32_t* flag) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t s = slot[i];
  if (s < 0) return;                                  // padding entry
  int bits = 0;
  if ((int64_t)s >= num_slots) bits |= 1;
  for (int j = i + 1; j < n; ++j)
    if (slot[j] == s) { bits |= 2; break; }
  if (bits) atomicOr(flag, bits);
}

hipError_t launch_validate_slots(const int32_t* slot, int n, int64_t num_slots, int32_t* flag,
                                 hipStream_t stream) {
  // A fill kernel rather than hipMemsetAsync keeps the pair graph-capturable.
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, stream, flag);
  if (n > 0)
    hipLaunchKernelGGL(validate_slots_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, slot,
                       n, num_slots, flag);
  return hipGetLastError();
}

}  // namespace gdn
