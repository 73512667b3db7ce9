// k_read.hip -- libtsel_probe.so: a read-only streaming kernel that measures
// the HBM read rate this GPU reaches in practice, reported beside the
// kernels' roofline fractions (the method's bound is the memory bandwidth,
// and the published peak is not reachable by any read).  Not part of
// libtsel.so.
//
// Every lane reads 16-byte words at a stride of the whole grid, four in
// flight, and folds them with xor; a fold that equals a fixed odd constant
// (which real data need not produce) is stored, so no load can be dropped.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tsel_probe.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_read(const uint4 *p, size_t n, uint32_t *out) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^
           (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;
}

}  // namespace

extern "C" int tsel_probe_read(const void *src, size_t bytes, int blocks, uint32_t *out,
                               void *stream) {
  if (!src || !out || bytes % 16 != 0 || blocks < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(src), bytes / 16, out);
  return (int)hipGetLastError();
}
