// k_vkey.hpp -- 16-bit value keys of bf16 scores, shared by the kernels that
// count a bf16 row into one histogram bin per value (k_vres, and the streamed
// histogram pass of k_full), and the removal of killed elements from a chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsel_internal.hpp"

namespace tsel {

// Scores as 16-bit keys whose integer order is the score order, with every
// score of magnitude at most 2^-kZoneExp on one of two keys: 0x7FFF (-0 and
// the negative ones) and 0x8000 (+0 and the positive ones).  From a bf16
// pattern u: t = max(|u| - Z, 0) with Z the magnitude bits of 2^-kZoneExp,
// then 0x8000 + t for a positive u and 0x7FFF - t for a negative one.
constexpr uint32_t kZoneMag = (uint32_t)(127 - kZoneExp) << 7;
constexpr uint32_t kKeyZoneNeg = 0x7FFFu, kKeyZonePos = 0x8000u;
constexpr uint32_t kKeyLowFinite = 0x7FFFu - (0x7F7Fu - kZoneMag);  // key of -max finite

__device__ __forceinline__ uint32_t vkey(uint32_t u) {
  const uint32_t m = u & 0x7FFFu;
  const uint32_t t = m > kZoneMag ? m - kZoneMag : 0u;
  return (u & 0x8000u) ? kKeyZoneNeg - t : kKeyZonePos + t;
}
// The bf16 value of a key off the two near-zero keys.
__device__ __forceinline__ float vkey_value(uint32_t k) {
  const uint32_t u = k > kKeyZonePos ? k - kKeyZonePos + kZoneMag
                                     : 0x8000u | (kKeyZoneNeg - k + kZoneMag);
  return __uint_as_float(u << 16);
}
// vkey without a select: the pattern in the low 16 bits of hw (the bits
// above are ignored); t: the clamped magnitude (0 on the near-zero keys).
__device__ __forceinline__ uint32_t vkey_t(uint32_t hw, uint32_t &t) {
  const uint32_t m = hw & 0x7FFFu;
  t = m > kZoneMag ? m - kZoneMag : 0u;
  return (t ^ (0u - ((hw >> 15) & 1u))) + 0x8000u;  // 0x8000 + t, or 0x7FFF - t
}
// Key of the largest bf16 value not above y (y not NaN; -0 counts as +0).
__device__ __forceinline__ uint32_t vkey_floor(float y) {
  uint32_t u = __float_as_uint(y + 0.0f);
  if ((u & 0x80000000u) && (u & 0xFFFFu)) u += 0x10000u;  // negative: away from zero
  return vkey(u >> 16);
}

// Removed elements of a chunk (kill bit j for element j) become -inf: for
// word q, bits 2q and 2q + 1 are shifted to the sign bit of each half and
// spread over it (two packed shifts, written out so that the compiler keeps
// them rather than a compare and select per half).
__device__ __forceinline__ uint4 vkill(uint4 c, uint32_t kb, uint32_t ninf) {
  const uint32_t kbp = (kb & 0xFFu) | ((kb & 0xFEu) << 15);  // bits 2q | bits 2q + 1 << 16
  uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t m;
    asm("v_pk_lshlrev_b16 %0, %1, %2 op_sel_hi:[0,1]\n\t"
        "v_pk_ashrrev_i16 %0, 15, %0 op_sel_hi:[0,1]"
        : "=&v"(m)
        : "n"(15 - 2 * q), "v"(kbp));
    w[q] = (m & ninf) | (~m & w[q]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace tsel
