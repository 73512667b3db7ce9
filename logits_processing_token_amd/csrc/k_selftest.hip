// k_selftest.hip -- an on-device check of the one hardware property the full
// sampling path relies on beyond IEEE arithmetic: the exp2 instruction
// (v_exp_f32) is monotone non-decreasing, so that mass-histogram bins are
// intervals of scores.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsel_device.hpp"
#include "tsel_internal.hpp"

namespace tsel {

// Count ordered keys k in [k0, k1) with exp2(x(k + 1)) < exp2(x(k)).
__global__ __launch_bounds__(256) void k_exp2_monotone(uint32_t k0, uint32_t k1,
                                                       unsigned long long *violations) {
  const uint64_t n = (uint64_t)k1 - k0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  unsigned long long v = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t k = k0 + (uint32_t)i;
    const float a = __builtin_amdgcn_exp2f(unordered_f32(k));
    const float b = __builtin_amdgcn_exp2f(unordered_f32(k + 1));
    v += b < a;
  }
  if (v) atomicAdd(violations, v);
}

hipError_t launch_exp2_monotone(uint32_t k0, uint32_t k1, unsigned long long *violations,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_exp2_monotone, dim3(8192), dim3(256), 0, s, k0, k1, violations);
  return hipGetLastError();
}

}  // namespace tsel
