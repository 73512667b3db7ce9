// k_exp2.hip -- libtsel_probe.so: an on-device check of the one hardware
// property the full sampling path relies on beyond IEEE arithmetic: the exp2
// instruction (v_exp_f32) is monotone non-decreasing, so that histogram bins
// of exp2 masses are intervals of scores.  Not part of libtsel.so.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "tsel_probe.h"

namespace {

// Binary32 from its order-preserving key (negative values reversed below the
// positive ones).
__device__ __forceinline__ float from_key(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Count keys k in [k0, k1) with exp2(x(k + 1)) < exp2(x(k)).
__global__ __launch_bounds__(256) void k_exp2_monotone(uint32_t k0, uint32_t k1,
                                                       unsigned long long *violations) {
  const uint64_t n = (uint64_t)k1 - k0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  unsigned long long v = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t k = k0 + (uint32_t)i;
    const float a = __builtin_amdgcn_exp2f(from_key(k));
    const float b = __builtin_amdgcn_exp2f(from_key(k + 1));
    v += b < a;
  }
  if (v) atomicAdd(violations, v);
}

uint32_t to_key(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  if (u == 0x80000000u) u = 0u;  // -0 and +0 are one point
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace

extern "C" int tsel_probe_exp2_monotone(float lo, float hi, unsigned long long *violations,
                                        void *stream) {
  if (!violations || !(lo <= hi)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_exp2_monotone, dim3(8192), dim3(256), 0,
                     static_cast<hipStream_t>(stream), to_key(lo), to_key(hi), violations);
  return (int)hipGetLastError();
}
