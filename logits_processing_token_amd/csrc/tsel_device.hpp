// tsel_device.hpp -- wave64 / workgroup building blocks shared by the tsel
// kernels (gfx950, CDNA4).  Device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsel {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Scores as ordered integer keys.
//
// ordered_f32 maps binary32 values to uint32 so that the integer order is the
// float order for every non-NaN value; -0.0 is first turned into +0.0 so that
// the two zeros compare equal, as they do as floats.
__device__ __forceinline__ uint32_t ordered_f32(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unordered_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Selection key of (score, id): a larger key is a larger score, and among
// equal scores the lower id.  0 is below every key of a real element.
__device__ __forceinline__ uint64_t sel_key(float x, uint32_t idx) {
  return ((uint64_t)ordered_f32(x) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) {
  return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu);
}
__device__ __forceinline__ float key_score(uint64_t k) {
  return unordered_f32((uint32_t)(k >> 32));
}

// bf16 bit patterns -> binary32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// e^d in binary64 for d <= 0 (-inf included: 0), by Cody and Waite's
// reduction and a Taylor polynomial: d = k ln2 + r with |r| <= ln2/2 (ln2
// split in two so that k * ln2_hi is exact), e^r by its Taylor series through
// r^13 (the next term is below 2^-57 of the sum), scaled by 2^k.  Within a
// unit in the last place of the exact value; no branch and a third of the
// operations of the general exp, for sums over every element of a row.
// (d is clamped at -746, where 2^k underflows to 0.)
__device__ __forceinline__ double exp_nonpos(double d) {
  d = fmax(d, -746.0);
  const double kInvLn2 = 1.4426950408889634074;
  const double kLn2Hi = 0x1.62e42fee00000p-1, kLn2Lo = 0x1.a39ef35793c76p-33;
  const double k = rint(d * kInvLn2);
  const double r = fma(-k, kLn2Lo, fma(-k, kLn2Hi, d));
  double p = 1.0 / 6227020800.0;             // 1/13!
  p = fma(p, r, 1.0 / 479001600.0);          // 1/12!
  p = fma(p, r, 1.0 / 39916800.0);           // 1/11!
  p = fma(p, r, 1.0 / 3628800.0);            // 1/10!
  p = fma(p, r, 1.0 / 362880.0);             // 1/9!
  p = fma(p, r, 1.0 / 40320.0);              // 1/8!
  p = fma(p, r, 1.0 / 5040.0);               // 1/7!
  p = fma(p, r, 1.0 / 720.0);                // 1/6!
  p = fma(p, r, 1.0 / 120.0);                // 1/5!
  p = fma(p, r, 1.0 / 24.0);                 // 1/4!
  p = fma(p, r, 1.0 / 6.0);                  // 1/3!
  p = fma(p, r, 0.5);                        // 1/2!
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, (int)k);
}

// Repetition penalty of a seen id, as in Python transformers: a negative
// score is multiplied by p, any other is divided by p (IEEE, round to
// nearest even; HIP keeps binary32 division correctly rounded by default).
__device__ __forceinline__ float penalize(float x, float p) {
  return x < 0.0f ? x * p : x / p;
}

// ---------------------------------------------------------------------------
// Values every lane of the wave holds alike (read from LDS, say) moved into
// scalar registers, which frees the vector registers they would occupy.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uni(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ float uni(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ __forceinline__ uint64_t uni(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double uni(double v) {
  return __longlong_as_double((long long)uni((uint64_t)__double_as_longlong(v)));
}

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes, by data-parallel lane moves (no
// LDS round trip): shifts by 1, 2, 4 and 8 within each row of 16 lanes,
// then the last lane of row 0 broadcast into row 1 and of row 2 into row 3,
// then lane 31 into rows 2 and 3.  (Lanes a move does not reach add 0.)
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

__device__ __forceinline__ double wave_incl_scan_f64(double v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    double w = __shfl_up(v, o, kWave);
    if (lane >= o) v += w;
  }
  return v;
}

// The same by row moves: each step moves the two halves of a double.
template <int CTRL, int ROWS, bool BC>
__device__ __forceinline__ double dpp_move_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROWS, 0xF, BC);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROWS, 0xF, BC);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

__device__ __forceinline__ double wave_incl_scan_f64_dpp(double v) {
  v += dpp_move_f64<0x111, 0xF, true>(v);   // row_shr:1
  v += dpp_move_f64<0x112, 0xF, true>(v);   // row_shr:2
  v += dpp_move_f64<0x114, 0xF, true>(v);   // row_shr:4
  v += dpp_move_f64<0x118, 0xF, true>(v);   // row_shr:8
  v += dpp_move_f64<0x142, 0xA, false>(v);  // row_bcast:15
  v += dpp_move_f64<0x143, 0xC, false>(v);  // row_bcast:31
  return v;
}

// Suffix sums within the wave (lane l gets the sum over lanes >= l): row
// moves to the left within each row of 16 lanes, then the totals of the rows
// above added from scalar registers.
__device__ __forceinline__ double wave_suffix_scan_f64_dpp(double v) {
  v += dpp_move_f64<0x101, 0xF, true>(v);  // row_shl:1
  v += dpp_move_f64<0x102, 0xF, true>(v);  // row_shl:2
  v += dpp_move_f64<0x104, 0xF, true>(v);  // row_shl:4
  v += dpp_move_f64<0x108, 0xF, true>(v);  // row_shl:8
  // (the first lane of row r now holds row r's total)
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  auto lane_value = [&](int l) {
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, l);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), l);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
  };
  const double t3 = lane_value(48), t2 = lane_value(32), t1 = lane_value(16);
  const double s3 = t3, s2 = t2 + t3, s1 = t1 + s2;
  const int row = (threadIdx.x & (kWave - 1)) >> 4;
  return v + (row == 0 ? s1 : row == 1 ? s2 : row == 2 ? s3 : 0.0);
}

// Maximum over the wave by row moves (quad swaps, half-row and row mirrors,
// then the row broadcasts), read from the last lane into a scalar register.
__device__ __forceinline__ float wave_max_f32_uni(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x140, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}
__device__ __forceinline__ uint32_t wave_max_u32_uni(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// ---------------------------------------------------------------------------
// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every global load the wave has in flight; a kernel that stages
// data in LDS while its row is still arriving uses this one instead.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int NT>
__device__ __forceinline__ float block_max_f32_lds(float v, float *scratch) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_max_f32(v);
  lds_barrier();
  if (lane == 0) scratch[wid] = v;
  lds_barrier();
  v = lane < NW ? scratch[lane] : -INFINITY;
  return wave_max_f32(v);
}

// ---------------------------------------------------------------------------
// Workgroup reductions.  `scratch` holds at least one slot per wave; every
// thread of the workgroup must call; the result is returned to all threads.
template <int NT>
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t *scratch) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_max_u64(v);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  v = lane < NW ? scratch[lane] : 0ull;
  return wave_max_u64(v);
}

template <int NT>
__device__ __forceinline__ float block_max_f32(float v, float *scratch) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_max_f32(v);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  v = lane < NW ? scratch[lane] : -INFINITY;
  return wave_max_f32(v);
}

template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double *scratch) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_sum_f64(v);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  v = lane < NW ? scratch[lane] : 0.0;
  return wave_sum_f64(v);
}

template <int NT>
__device__ __forceinline__ int block_sum_i32(int v, int *scratch) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_sum_i32(v);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  v = lane < NW ? scratch[lane] : 0;
  return wave_sum_i32(v);
}

// Exclusive prefix sum over the workgroup in thread order; *total gets the
// sum of all values.  LDS_ONLY: barriers that do not wait for global loads.
template <int NT, bool LDS_ONLY = false>
__device__ __forceinline__ int block_excl_scan_i32(int v, int *scratch, int *total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  int incl = wave_incl_scan_i32(v);
  if (LDS_ONLY) lds_barrier(); else __syncthreads();
  if (lane == kWave - 1) scratch[wid] = incl;
  if (LDS_ONLY) lds_barrier(); else __syncthreads();
  int wsum = lane < NW ? scratch[lane] : 0;
  int wincl = wave_incl_scan_i32(wsum);
  int wbase = __shfl(wincl - wsum, wid, kWave);
  *total = __shfl(wincl, NW - 1, kWave);
  return wbase + incl - v;
}

}  // namespace tsel
