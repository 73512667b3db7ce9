// k_mask.hip -- bitmask of a list of single token ids: the static masks of
// the single-token bad words and of suppress_tokens, built once per group of
// rows ("Transmuter.Generation (transmuter v2.0.0)", section "Processors").

#include <hip/hip_runtime.h>

#include "tsel_internal.hpp"

namespace tsel {

constexpr int kMaskThreads = 1024;

// One workgroup: clear every word, then set one bit per listed id.
__global__ __launch_bounds__(kMaskThreads) void k_mask_build(int32_t V, const int32_t *ids,
                                                              int32_t n, uint32_t *mask) {
  const int words = (V + 31) / 32;
  for (int w = threadIdx.x; w < words; w += kMaskThreads) mask[w] = 0u;
  __threadfence();  // the clears reach L2 before any wave's atomics
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kMaskThreads) {
    const int v = ids[i];
    if (v >= 0 && v < V) atomicOr(&mask[v >> 5], 1u << (v & 31));
  }
}

hipError_t launch_mask_build(int32_t V, const int32_t *ids, int32_t n, uint32_t *mask,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_mask_build, dim3(1), dim3(kMaskThreads), 0, s, V, ids, n, mask);
  return hipGetLastError();
}

}  // namespace tsel
