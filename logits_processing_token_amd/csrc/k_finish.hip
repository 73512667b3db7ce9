// The end of one decode step, on the device: each row's emitted token and
// finished flag, so that a decode loop needs no host read per step
// ("Transmuter.Generation (transmuter v2.0.0)", function doc of generate/5:
// the on_token callback and the return value; mlxcel inference pipeline,
// decode loop: EOS detection and stopping).
//
// One lane per row; the stop ids are staged once per workgroup in LDS.
// Integer work only: each row reads 13 bytes and writes 5.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tsel_internal.hpp"

namespace tsel {

constexpr int kFinishThreads = 256;

__global__ __launch_bounds__(kFinishThreads) void k_finish(int32_t B, const int32_t *tokens,
                                                           const int32_t *lens,
                                                           const int32_t *max_lengths,
                                                           const int32_t *eos, int32_t n_eos,
                                                           uint8_t *finished, int32_t *out) {
  __shared__ int32_t stop[kMaxFinishEos];
  for (int i = threadIdx.x; i < n_eos; i += kFinishThreads) stop[i] = eos[i];
  __syncthreads();
  const int b = blockIdx.x * kFinishThreads + threadIdx.x;
  if (b >= B) return;
  const int32_t t = tokens[b];
  const uint8_t was = finished[b];
  int32_t emit = -1;
  uint8_t fin = 1;
  if (!was && t >= 0) {  // (a finished row, or one without a token, emits nothing)
    bool is_stop = false;
    for (int i = 0; i < n_eos; ++i) is_stop |= stop[i] == t;
    if (!is_stop) {  // (a stop id ends the row unemitted)
      emit = t;
      fin = (int64_t)lens[b] + 1 >= (int64_t)max_lengths[b] ? 1 : 0;
    }
  }
  out[b] = emit;
  finished[b] = fin;
}

hipError_t launch_finish(int32_t B, const int32_t *tokens, const int32_t *lens,
                         const int32_t *max_lengths, const int32_t *eos, int32_t n_eos,
                         uint8_t *finished, int32_t *out, hipStream_t s) {
  const int grid = (B + kFinishThreads - 1) / kFinishThreads;
  hipLaunchKernelGGL(k_finish, dim3(grid), dim3(kFinishThreads), 0, s, B, tokens, lens,
                     max_lengths, eos, n_eos, finished, out);
  return hipGetLastError();
}

}  // namespace tsel
