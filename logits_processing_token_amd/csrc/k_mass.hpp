// k_mass.hpp -- exact probability-mass bookkeeping shared by the sampling
// kernels (k_full, k_res): the mass of a score relative to a reference, its
// histogram bin, the exact mass of a bin, and the bisection over selection
// keys that decides top_p and the draw by re-reading the row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k_select_common.hpp"

namespace tsel {

// Histogram bin of a mass e >= 0 (its binary32 bits): the exponent and the
// top mantissa bits, offset so that bin 1 starts kBinBelow binades below the
// reference; bin 0 holds e == 0 and everything smaller, the last bin
// everything larger.
__device__ __forceinline__ int mass_bin(uint32_t bits, int shift, int base, int nb) {
  return min(max((int)(bits >> shift), base), base + nb - 1) - base;  // one v_med3_i32
}

// Exact sum of the masses of bin b from its (count, low-bit sum) word.  Bin
// 0 (removed ids and masses below the covered range) counts as 0.
__device__ __forceinline__ double bin_mass(uint64_t acc, int b, int shift, int base) {
  const uint64_t cnt = acc >> 40;
  if (b == 0 || cnt == 0) return 0.0;
  const uint64_t low = acc & ((1ull << 40) - 1);
  // The bin's smallest mass e_lo has the bin's top bits and zero low bits;
  // every member is e_lo + (its low bits) * ulp, ulp = 2^(exponent - 150).
  const uint32_t lo_bits = (uint32_t)(b + base) << shift;
  const double e_lo = (double)__uint_as_float(lo_bits);
  const int expo = (int)(lo_bits >> 23);  // binary32 exponent field, 1..254
  const double ulp = __longlong_as_double((long long)(expo - 150 + 1023) << 52);
  return (double)cnt * e_lo + (double)low * ulp;  // both products exact
}

// Mass of a final score y relative to the reference (cref = r log2 e); with
// a top_k, scores below its threshold t_y have none.  exp2(-inf) = 0, so
// removed ids (-inf) have none either.
template <bool TOPK = true>
__device__ __forceinline__ float mass_of(float y, float t_y, float cref) {
  const float e = __builtin_amdgcn_exp2f(fmaf(y, kLog2e, -cref));
  return TOPK ? ((y >= t_y) ? e : 0.0f) : e;
}

// ---------------------------------------------------------------------------
// Slow, general pieces: they re-read the row from memory.

// Exact k-th largest final score of the row (radix select over the stream).
template <int DT>
__device__ __forceinline__ float topk_threshold_stream(const SelectArgs &a, int row, const Lds &s,
                                                    RowShared &sh, int k_eff) {
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  const float T = a.temperature;
  const int n_list = sh.n_list;
  const bool dense_pen = sh.dense_pen != 0;
  const uint32_t tk = radix_kth_largest(
      [&](auto &&f) {
        stream_row<DT>(a, rowp, s, dense_pen, [&](int, float x) {
          const float y = (T != 1.0f) ? x / T : x;
          if (y > -INFINITY) f(ordered_f32(y));
        });
        for (int i = threadIdx.x; i < n_list; i += NT) {
          const float y = (T != 1.0f) ? s.list_val[i] / T : s.list_val[i];
          f(ordered_f32(y));
        }
      },
      k_eff, s.rhist, sh);
  return tk == 0u ? -INFINITY : unordered_f32(tk);
}

// Every id of the row that the kill mask keeps, one element per thread and
// step, straight from memory (few registers; for layouts whose list does not
// carry the row tail).
template <int DT, class F>
__device__ __forceinline__ void visit_plain(const SelectArgs &a, const char *rowp, const Lds &s, F &&f) {
  for (int v = threadIdx.x; v < a.V; v += NT)
    if (!bit_of(s.kmask, v)) f(v, Elem<DT>::load1(rowp, v));
}

// Mass of the elements (score >= t_y) whose selection key is >= q.  PLAIN:
// visit the row with visit_plain rather than the chunk stream.
template <int DT, bool PLAIN = false>
__device__ __forceinline__ double mass_key_ge(const SelectArgs &a, int row, const Lds &s,
                                          RowShared &sh, float t_y, float cref, uint64_t q) {
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  const float T = a.temperature;
  const int n_list = sh.n_list;
  double m = 0.0;
  auto body = [&](int v, float x) {
    const float y = (T != 1.0f) ? x / T : x;
    if (y > -INFINITY && y >= t_y && sel_key(y, (uint32_t)v) >= q) m += (double)mass_of(y, t_y, cref);
  };
  if (PLAIN) visit_plain<DT>(a, rowp, s, body);
  else stream_row<DT>(a, rowp, s, sh.dense_pen != 0, body);
  for (int i = threadIdx.x; i < n_list; i += NT) {
    const float y = (T != 1.0f) ? s.list_val[i] / T : s.list_val[i];
    if (y >= t_y && sel_key(y, (uint32_t)s.list_id[i]) >= q) m += (double)mass_of(y, t_y, cref);
  }
  return block_sum_f64<NT>(m, sh.red_f64);
}

// The token's log-probability over the final scores of its row
// ("Transmuter.Generation (transmuter v2.0.0)", "Log-probabilities"): the
// kept scores are those >= t_y whose selection key is >= kcut, each after
// temperature; the result is y_t - M - log(sum exp(y - M)) over them in
// binary64, rounded once (NaN when nothing is kept).  One more pass over
// the row (PLAIN: visit_plain rather than the chunk stream) and the list;
// the token's own final score is picked up on the way.
template <int DT, bool PLAIN = false>
__device__ __forceinline__ float kept_logprob(const SelectArgs &a, int row, const Lds &s,
                                              RowShared &sh, float t_y, uint64_t kcut,
                                              int token) {
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  const float T = a.temperature;
  const int n_list = sh.n_list;
  LseAcc acc;
  float yt = -INFINITY;
  auto body = [&](int v, float y) {
    if (v == token) yt = y;
    if (y > -INFINITY && y >= t_y && sel_key(y, (uint32_t)v) >= kcut) acc.add(y);
  };
  if (PLAIN) visit_plain<DT>(a, rowp, s, [&](int v, float x) { body(v, (T != 1.0f) ? x / T : x); });
  else stream_row<DT>(a, rowp, s, sh.dense_pen != 0,
                      [&](int v, float x) { body(v, (T != 1.0f) ? x / T : x); });
  for (int i = threadIdx.x; i < n_list; i += NT)
    body(s.list_id[i], (T != 1.0f) ? s.list_val[i] / T : s.list_val[i]);
  float M;
  double S;
  lse_join<NT>(acc, sh.red_f32, sh.red_f64, &M, &S);
  yt = block_max_f32<NT>(yt, sh.red_f32);
  if (!(M > -INFINITY) || !(yt > -INFINITY)) return lp_none();
  return (float)(((double)yt - (double)M) - log(S));
}

// Top_p cut and inverse-CDF draw by bisection over 64-bit selection keys.
// Returns the token; *kcut_out = smallest kept key.
template <int DT, bool PLAIN = false>
__device__ __forceinline__ int bisect_select(const SelectArgs &a, int row, const Lds &s,
                                          RowShared &sh, float t_y, float cref,
                                          uint64_t *kcut_out) {
  const double W = mass_key_ge<DT, PLAIN>(a, row, s, sh, t_y, cref, 1ull);
  const double pw = (double)a.top_p * W;
  uint64_t kcut = 0ull;
  double Wp = W;
  if (a.top_p < 1.0f && pw <= W) {
    // kept iff the mass of larger keys is < pW: kcut is the smallest q with
    // mass(key > q) = mass(key >= q + 1) < pW.  No element has key ~0.
    uint64_t lo = 0ull, hi = ~0ull - 1ull;
    while (hi - lo > 1ull) {
      const uint64_t mid = lo + (hi - lo) / 2;
      if (mass_key_ge<DT, PLAIN>(a, row, s, sh, t_y, cref, mid + 1) < pw) hi = mid; else lo = mid;
    }
    kcut = hi;
    Wp = mass_key_ge<DT, PLAIN>(a, row, s, sh, t_y, cref, kcut);
  }
  const double target = (double)a.uniforms[row] * Wp;
  // the token's key is max{q >= kcut : mass(key >= q) > target}
  uint64_t lo = kcut, hi = ~0ull;
  if (mass_key_ge<DT, PLAIN>(a, row, s, sh, t_y, cref, lo) > target) {
    while (hi - lo > 1ull) {
      const uint64_t mid = lo + (hi - lo) / 2;
      if (mass_key_ge<DT, PLAIN>(a, row, s, sh, t_y, cref, mid) > target) lo = mid; else hi = mid;
    }
  } else {
    // rounding at the very end: the smallest kept key
    const char *rowp = a.logits + (int64_t)row * a.row_bytes;
    const float T = a.temperature;
    uint64_t best = 0ull;
    auto body = [&](int v, float x) {
      const float y = (T != 1.0f) ? x / T : x;
      if (y > -INFINITY && y >= t_y) {
        const uint64_t kk = sel_key(y, (uint32_t)v);
        if (kk >= kcut) best = max(best, ~kk);
      }
    };
    if (PLAIN) visit_plain<DT>(a, rowp, s, body);
    else stream_row<DT>(a, rowp, s, sh.dense_pen != 0, body);
    for (int i = threadIdx.x; i < sh.n_list; i += NT) {
      const float y = (T != 1.0f) ? s.list_val[i] / T : s.list_val[i];
      const uint64_t kk = sel_key(y, (uint32_t)s.list_id[i]);
      if (y >= t_y && kk >= kcut) best = max(best, ~kk);
    }
    best = block_max_u64<NT>(best, sh.red_u64);
    lo = ~best;
  }
  *kcut_out = kcut;
  return (int)key_index(lo);
}

}  // namespace tsel
