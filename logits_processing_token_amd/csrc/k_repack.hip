// k_repack.hip -- rows whose byte stride is not a multiple of 16 copied into
// rows that are (the kernels read rows in 16-byte units from 16-byte aligned
// starts).  One thread writes one 16-byte unit of a destination row: the
// row's elements there, read one by one at their element alignment, and
// zeros past the row's end.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsel_internal.hpp"

namespace tsel {
namespace {

template <int ES>
__global__ __launch_bounds__(256) void k_repack(const unsigned char *src, int64_t src_stride,
                                                unsigned char *dst, int64_t dst_stride, int32_t V,
                                                int32_t units, int32_t ublocks) {
  // (one block: 256 units of one row; the row's blocks are consecutive)
  const int64_t row = blockIdx.x / (uint32_t)ublocks;
  const int u = (int)(blockIdx.x - row * ublocks) * 256 + threadIdx.x;
  if (u >= units) return;
  const unsigned char *s = src + row * src_stride * ES;
  constexpr int E = 16 / ES;  // elements per unit
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int v = u * E + j;
    if (v >= V) break;
    if (ES == 2) {
      const uint32_t x = *reinterpret_cast<const uint16_t *>(s + 2 * (int64_t)v);
      w[j >> 1] |= x << (16 * (j & 1));
    } else {
      w[j] = *reinterpret_cast<const uint32_t *>(s + 4 * (int64_t)v);
    }
  }
  reinterpret_cast<uint4 *>(dst + row * dst_stride * ES)[u] = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

hipError_t launch_repack(const void *src, int32_t dtype, int64_t src_stride, void *dst,
                         int64_t dst_stride, int32_t rows, int32_t V, hipStream_t s) {
  const int es = dtype == 1 ? 2 : 4;
  const int32_t units = (int32_t)(dst_stride * es / 16);
  const int32_t ublocks = (units + 255) / 256;
  if ((int64_t)rows * ublocks > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)(rows * ublocks));
  if (es == 2)
    hipLaunchKernelGGL(k_repack<2>, grid, dim3(256), 0, s, static_cast<const unsigned char *>(src),
                       src_stride, static_cast<unsigned char *>(dst), dst_stride, V, units, ublocks);
  else
    hipLaunchKernelGGL(k_repack<4>, grid, dim3(256), 0, s, static_cast<const unsigned char *>(src),
                       src_stride, static_cast<unsigned char *>(dst), dst_stride, V, units, ublocks);
  return hipGetLastError();
}

}  // namespace tsel
