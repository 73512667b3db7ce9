// k_select.hip -- fused per-row token selection for gfx950 (CDNA4).
//
// One workgroup of 1024 threads (16 wave64s) owns one row of the [B, V]
// logits of a decode step and runs the whole chain there, reading every
// logit from HBM once (a coalesced 16-byte-per-lane stream):
//
//   staging   history -> on-chip "seen" bitmask; no-repeat n-gram bans from a
//             scan of the history; static bad-word / suppress /
//             begin-suppress bitmasks, the eos set and the n-gram bans folded
//             into one on-chip "kill" bitmask; the distinct seen ids that are
//             not killed become a short list whose logits are gathered and
//             penalized once.  The dense stream then treats seen ids as
//             killed, so the per-element work is a bit test.
//   greedy    argmax over the stream (lowest id among equal scores).
//   top_k     a candidate filter: a running k-th-largest threshold decides
//             which logits enter an on-chip candidate buffer; the exact top_k,
//             top_p and the inverse-CDF draw then run on the candidates.
//   full      sampling without top_k (or a top_k the buffer cannot hold): the
//             row stays in registers when it fits, else it is re-read.  Row
//             max, then exp-mass histogram over value bins below the max;
//             the bin holding the top_p boundary and the bin holding the
//             sample are collected on chip and ordered exactly by
//             (score desc, id asc); a bisection over keys covers bins too
//             large to collect.
//
// Processor semantics and order: "Transmuter.Generation (transmuter v2.0.0)",
// module doc (order), "Lengths" (length rules), "Processors" (static masks),
// "Batches" (padding rows), generate/5 (token -1).  Sampling by the inverse
// CDF of a caller uniform in (score desc, id asc) order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsel_device.hpp"
#include "tsel_internal.hpp"

namespace tsel {

constexpr int NT = kSelectThreads;
constexpr int NW = NT / kWave;
constexpr int U = 8;                 // 16-byte chunks in flight per lane when streaming
constexpr float kBinRange = 32.0f;   // nats below the row max covered by the mass histogram
constexpr uint32_t kNoDigit = 0xFFFFFFFFu;

template <int DT>
struct Elem;
template <>
struct Elem<0> {  // binary32
  static constexpr int EPC = 4;
  __device__ static __forceinline__ float get(const uint4 &c, int j) {
    return __uint_as_float(j == 0 ? c.x : j == 1 ? c.y : j == 2 ? c.z : c.w);
  }
  __device__ static __forceinline__ float load1(const char *row, int v) {
    return reinterpret_cast<const float *>(row)[v];
  }
};
template <>
struct Elem<1> {  // bf16
  static constexpr int EPC = 8;
  __device__ static __forceinline__ float get(const uint4 &c, int j) {
    uint32_t w = (j >> 1) == 0 ? c.x : (j >> 1) == 1 ? c.y : (j >> 1) == 2 ? c.z : c.w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  __device__ static __forceinline__ float load1(const char *row, int v) {
    uint32_t h = reinterpret_cast<const uint16_t *>(row)[v];
    return __uint_as_float(h << 16);
  }
};

struct RowShared {
  uint64_t red_u64[NW];
  double red_f64[NW];
  float red_f32[NW];
  int red_i32[NW];
  int n_list;      // entries of the sparse list (seen-and-alive ids, then the row tail)
  int n_seen;      // of which the first n_seen are seen ids
  int dense_pen;   // 1: too many distinct seen ids; the stream penalizes them itself
  int count;       // top_k candidates in the buffer
  int overflow;    // the candidate buffer could not hold the candidates
  uint32_t digit;  // radix select result of the current pass
  int krem;
  float tau_x;     // filter on pre-temperature scores for the candidate buffer
  int token;
  uint64_t kcut;   // smallest selection key kept by top_p (0 = no cut)
  float t_y;       // top_k threshold on the final scores (-inf = none)
  double w_sum;
  double a0;
  int bin_p, bin_u;
  int n_coll;
  double wprime;
  int found;
};

__device__ __forceinline__ uint4 load16(const char *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

// Kill / seen bits of chunk g: bit j covers element g * EPC + j.
template <int DT>
__device__ __forceinline__ uint32_t chunk_bits(const uint8_t *m, int g) {
  if (DT == 1) return m[g];
  return (m[g >> 1] >> ((g & 1) * 4)) & 0xFu;
}

__device__ __forceinline__ bool bit_of(const uint32_t *m, int v) {
  return (m[v >> 5] >> (v & 31)) & 1u;
}

// Smallest binary32 x with RN(x / T) >= RN(tau / T): the pre-temperature
// threshold that admits every score the temperature maps onto the same value
// as tau (division by T > 0 is monotone but can merge neighbours).
__device__ float pre_temperature_floor(float tau, float T) {
  if (T == 1.0f || tau == -INFINITY) return tau;
  const float t = tau / T;
  uint32_t hi = ordered_f32(tau), lo = 0;  // f(unordered(hi)) >= t
  while (hi - lo > 1) {
    uint32_t mid = lo + (hi - lo) / 2;
    if (unordered_f32(mid) / T >= t) hi = mid; else lo = mid;
  }
  return unordered_f32(hi);
}

// k-th largest of a multiset of ordered keys, by an LDS radix select over
// four 8-bit digits.  visit(f) must call f(key) once for every element (from
// all threads together).  Returns 0 when the multiset has fewer than k
// elements.  Every thread of the workgroup must call.
template <class Visit>
__device__ uint32_t radix_kth_largest(Visit &&visit, int k, uint32_t *hist, RowShared &sh) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    visit([&](uint32_t ok) {
      if ((ok & pmask) == prefix) atomicAdd(&hist[(ok >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (tid < kWave) {
      const int l = tid;
      uint32_t c0 = hist[255 - 4 * l], c1 = hist[254 - 4 * l], c2 = hist[253 - 4 * l],
               c3 = hist[252 - 4 * l];
      int s = (int)(c0 + c1 + c2 + c3);
      int incl = wave_incl_scan_i32(s);
      int excl = incl - s;
      if (excl < krem && krem <= incl) {
        int r = krem - excl;
        uint32_t d;
        if ((int)c0 >= r) d = 255 - 4 * l;
        else if ((int)(c0 + c1) >= r) { d = 254 - 4 * l; r -= (int)c0; }
        else if ((int)(c0 + c1 + c2) >= r) { d = 253 - 4 * l; r -= (int)(c0 + c1); }
        else { d = 252 - 4 * l; r -= (int)(c0 + c1 + c2); }
        sh.digit = d;
        sh.krem = r;
      }
      if (l == kWave - 1 && incl < krem) sh.digit = kNoDigit;
    }
    __syncthreads();
    const uint32_t d = sh.digit;
    if (d == kNoDigit) return 0u;
    prefix |= d << shift;
    pmask |= 0xFFu << shift;
    krem = sh.krem;
    __syncthreads();
  }
  return prefix;
}

// In-place ordering of n selection keys (descending) in LDS by ranks; keys are
// distinct (they carry the id).  vals move with their keys.
template <typename TV>
__device__ void rank_sort_desc(uint64_t *keys, TV *vals, int n, uint64_t *tmpk, TV *tmpv) {
  const int tid = threadIdx.x;
  for (int i = tid; i < n; i += NT) {
    uint64_t ki = keys[i];
    int r = 0;
    for (int j = 0; j < n; ++j) r += keys[j] > ki;
    tmpk[r] = ki;
    tmpv[r] = vals[i];
  }
  __syncthreads();
  for (int i = tid; i < n; i += NT) {
    keys[i] = tmpk[i];
    vals[i] = tmpv[i];
  }
  __syncthreads();
}

template <int DT, int RES>
__global__ __launch_bounds__(NT, 1) void k_select(SelectArgs a) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RowShared sh;
  uint32_t *kmask = reinterpret_cast<uint32_t *>(smem);
  uint32_t *smask = reinterpret_cast<uint32_t *>(smem + a.off_smask);
  int32_t *list_id = reinterpret_cast<int32_t *>(smem + a.off_list_id);
  float *list_val = reinterpret_cast<float *>(smem + a.off_list_val);
  uint32_t *rhist = reinterpret_cast<uint32_t *>(smem + a.off_area);  // 256 words
  unsigned char *area = smem + a.off_area + 1024;
  const uint8_t *kbytes = reinterpret_cast<const uint8_t *>(kmask);
  const uint8_t *sbytes = reinterpret_cast<const uint8_t *>(smask);

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int V = a.V;
  const int NG = V / EPC;          // whole 16-byte chunks
  const int Vvec = NG * EPC;       // ids [Vvec, V) form the row tail
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  const int L = a.lens[row];
  const int P = a.lens[a.B + row];
  const int M = a.lens[2 * a.B + row];
  float *outp = a.out_processed ? a.out_processed + (int64_t)row * V : nullptr;

  // ---- padding row: no token ----------------------------------------------
  if (L <= 0) {
    if (tid == 0) a.out_tokens[row] = -1;
    if (outp)
      for (int v = tid; v < V; v += NT) outp[v] = -INFINITY;
    return;
  }
  const int new_tokens = L - P;
  const bool begin_active =
      a.begin_mask != nullptr && new_tokens == ((a.forced_bos >= 0 && P == 1) ? 1 : 0);

  // ---- forced rows: forced_bos at one token, forced_eos at max_length - 1 --
  int forced = -1;
  if (a.forced_bos >= 0 && L == 1) forced = a.forced_bos;
  if (a.forced_eos >= 0 && L == M - 1) forced = a.forced_eos;  // later processor wins
  if (forced >= 0) {
    bool alive = forced < V;
    if (alive && a.sup_mask && bit_of(a.sup_mask, forced)) alive = false;
    if (alive && begin_active && bit_of(a.begin_mask, forced)) alive = false;
    if (tid == 0) a.out_tokens[row] = alive ? forced : 0;
    if (outp)
      for (int v = tid; v < V; v += NT) outp[v] = (alive && v == forced) ? 0.0f : -INFINITY;
    return;
  }

  const bool sampling = a.do_sample != 0;
  const float T = a.temperature;
  const bool use_topk = sampling && a.top_k > 0 && min(a.top_k, V) * 4 <= a.tcap;
  const bool full_first = sampling && !use_topk;

  // The whole row in registers when it fits and the row goes straight to the
  // full path: issue the loads first so that they fly during staging.
  uint4 reg[RES > 0 ? RES : 1];
  if (RES > 0 && full_first) {
#pragma unroll
    for (int i = 0; i < RES; ++i) {
      const int g = tid + i * NT;
      if (g < NG) reg[i] = load16(rowp + (int64_t)g * 16);
    }
  }

  // ---- staging ---------------------------------------------------------------
  const int mw = a.mw;
  for (int w = tid; w < mw; w += NT) {
    kmask[w] = 0u;
    smask[w] = 0u;
  }
  if (tid == 0) {
    sh.count = 0;
    sh.overflow = 0;
  }
  __syncthreads();
  const int32_t *h = a.hist + (int64_t)row * a.hist_stride;
  for (int i = tid; i < L; i += NT) {
    const int v = h[i];
    if (v >= 0 && v < V) atomicOr(&smask[v >> 5], 1u << (v & 31));
  }
  const int n = a.ngram;
  if (n > 0 && L >= n) {
    // Window i of the history bans its last id when its first n-1 ids equal
    // the last n-1 ids of the history.
    const int32_t *tail = h + (L - n + 1);
    for (int i = tid; i + n <= L; i += NT) {
      bool match = true;
      for (int j = 0; j < n - 1; ++j)
        if (h[i + j] != tail[j]) { match = false; break; }
      const int t = h[i + n - 1];
      if (match && t >= 0 && t < V) atomicOr(&kmask[t >> 5], 1u << (t & 31));
    }
  }
  const bool minlen_active = a.min_new > 0 ? (new_tokens < a.min_new)
                                           : (a.min_length > 0 && L < a.min_length);
  if (minlen_active && tid < a.n_eos) {
    const int e = a.eos[tid];
    if (e >= 0 && e < V) atomicOr(&kmask[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  // Fold the static masks in; count the seen ids that stay alive.
  const int wpt = (mw + NT - 1) / NT;  // words per thread, contiguous
  int my_cnt = 0;
  for (int q = 0; q < wpt; ++q) {
    const int w = tid * wpt + q;
    if (w < mw) {
      uint32_t k = kmask[w];
      if (a.bad_mask) k |= a.bad_mask[w];
      if (a.sup_mask) k |= a.sup_mask[w];
      if (begin_active) k |= a.begin_mask[w];
      kmask[w] = k;
      my_cnt += __popc(smask[w] & ~k);
    }
  }
  int n_seen_total = 0;
  const int my_off = block_excl_scan_i32<NT>(my_cnt, sh.red_i32, &n_seen_total);
  const int ntail = V - Vvec;
  const bool dense_pen = n_seen_total > a.lcap - 8;
  if (!dense_pen) {
    int o = my_off;
    for (int q = 0; q < wpt; ++q) {
      const int w = tid * wpt + q;
      if (w < mw) {
        uint32_t bits = smask[w] & ~kmask[w];
        while (bits) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1;
          list_id[o++] = w * 32 + b;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int o = dense_pen ? 0 : n_seen_total;
    sh.n_seen = o;
    for (int v = Vvec; v < V; ++v) {
      const bool killed = bit_of(kmask, v) || (!dense_pen && bit_of(smask, v));
      if (!killed) list_id[o++] = v;
    }
    sh.n_list = o;
    sh.dense_pen = dense_pen ? 1 : 0;
  }
  (void)ntail;
  __syncthreads();
  if (!dense_pen)  // the stream treats seen ids as killed; the list carries them
    for (int w = tid; w < mw; w += NT) kmask[w] |= smask[w];
  const int n_list = sh.n_list;
  // Gather the listed logits (the row's lines are in flight or in L2).
  for (int i = tid; i < n_list; i += NT) {
    const int v = list_id[i];
    float x = E::load1(rowp, v);
    if (bit_of(smask, v)) x = penalize(x, a.rep);
    list_val[i] = x;
  }
  __syncthreads();

  const float rep = a.rep;
  // Visit every dense element of this lane once, in increasing id order:
  // f(id, x, alive) with x after the penalty (when the stream applies it).
  auto stream_dense = [&](auto &&f) {
    for (int g0 = tid; g0 < NG; g0 += NT * U) {
      uint4 c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = g0 + u * NT;
        if (g < NG) c[u] = load16(rowp + (int64_t)g * 16);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = g0 + u * NT;
        if (g < NG) {
          const uint32_t kb = chunk_bits<DT>(kbytes, g);
          const uint32_t sb = dense_pen ? chunk_bits<DT>(sbytes, g) : 0u;
#pragma unroll
          for (int j = 0; j < EPC; ++j) {
            float x = E::get(c[u], j);
            if ((sb >> j) & 1u) x = penalize(x, rep);
            f(g * EPC + j, x, !((kb >> j) & 1u));
          }
        }
      }
    }
  };

  // ======================= greedy =======================================
  if (!sampling) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    stream_dense([&](int v, float x, bool alive) {
      if (alive && x > bv) { bv = x; bi = v; }
      if (outp) outp[v] = alive ? x : -INFINITY;
    });
    if (outp)
      for (int v = Vvec + tid; v < V; v += NT) outp[v] = -INFINITY;
    uint64_t key = bi == 0x7FFFFFFF ? 0ull : sel_key(bv, (uint32_t)bi);
    for (int i = tid; i < n_list; i += NT) {
      const uint64_t k2 = sel_key(list_val[i], (uint32_t)list_id[i]);
      key = k2 > key ? k2 : key;
    }
    key = block_max_u64<NT>(key, sh.red_u64);
    if (tid == 0) a.out_tokens[row] = key == 0ull ? 0 : (int)key_index(key);
    if (outp) {
      __syncthreads();
      for (int i = tid; i < n_list; i += NT) outp[list_id[i]] = list_val[i];
    }
    return;
  }

  // ======================= sampling =====================================
  const double p_top = (double)a.top_p;
  const bool use_top_p = a.top_p < 1.0f;
  const double u = (double)a.uniforms[row];
  const int k_eff = a.top_k > 0 ? min(a.top_k, V) : 0;
  bool done = false;

  if (use_topk) {
    // ---------------- candidate filter -----------------------------------
    float *cx = reinterpret_cast<float *>(area);
    int32_t *ci = reinterpret_cast<int32_t *>(area + 4 * a.tcap);
    const int tcap = a.tcap;
    auto append = [&](int v, float x) {
      const int slot = atomicAdd(&sh.count, 1);
      if (slot < tcap) { cx[slot] = x; ci[slot] = v; }
      else sh.overflow = 1;
    };
    // Threshold from the first tile: the k-th largest alive score of the
    // first U chunks of every lane (a lower bound of the row's).
    uint4 c0[U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int g = tid + uu * NT;
      if (g < NG) c0[uu] = load16(rowp + (int64_t)g * 16);
    }
    auto first_tile = [&](auto &&f) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int g = tid + uu * NT;
        if (g < NG) {
          const uint32_t kb = chunk_bits<DT>(kbytes, g);
          const uint32_t sb = dense_pen ? chunk_bits<DT>(sbytes, g) : 0u;
#pragma unroll
          for (int j = 0; j < EPC; ++j) {
            float x = E::get(c0[uu], j);
            if ((sb >> j) & 1u) x = penalize(x, rep);
            if (!((kb >> j) & 1u)) f(g * EPC + j, x);
          }
        }
      }
    };
    const uint32_t t0 = radix_kth_largest(
        [&](auto &&f) { first_tile([&](int, float x) { f(ordered_f32(x)); }); }, k_eff, rhist, sh);
    float tau = t0 == 0u ? -INFINITY : unordered_f32(t0);
    if (tid == 0) sh.tau_x = pre_temperature_floor(tau, T);
    __syncthreads();
    float flt = sh.tau_x;
    first_tile([&](int v, float x) {
      if (x >= flt) append(v, x);
    });
    for (int i = tid; i < n_list; i += NT)
      if (list_val[i] >= flt) append(list_id[i], list_val[i]);
    __syncthreads();
    // Remaining tiles; prune the buffer at tile ends when it is half full.
    for (int t0g = NT * U; t0g < NG && !sh.overflow; t0g += NT * U) {
      uint4 c[U];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int g = t0g + tid + uu * NT;
        if (g < NG) c[uu] = load16(rowp + (int64_t)g * 16);
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int g = t0g + tid + uu * NT;
        if (g < NG) {
          const uint32_t kb = chunk_bits<DT>(kbytes, g);
          const uint32_t sb = dense_pen ? chunk_bits<DT>(sbytes, g) : 0u;
#pragma unroll
          for (int j = 0; j < EPC; ++j) {
            float x = E::get(c[uu], j);
            if ((sb >> j) & 1u) x = penalize(x, rep);
            if (!((kb >> j) & 1u) && x >= flt) append(g * EPC + j, x);
          }
        }
      }
      __syncthreads();
      if (!sh.overflow && sh.count > tcap / 2) {
        // Prune: new threshold = k-th largest in the buffer.
        const int cnt = sh.count;
        const uint32_t tk = radix_kth_largest(
            [&](auto &&f) {
              for (int i = tid; i < cnt; i += NT) f(ordered_f32(cx[i]));
            },
            k_eff, rhist, sh);
        if (tid == 0) sh.tau_x = pre_temperature_floor(tk == 0u ? -INFINITY : unordered_f32(tk), T);
        __syncthreads();
        flt = sh.tau_x;
        // Compact: each thread moves the entries it owns.
        constexpr int kPer = 8;
        float mx[kPer];
        int mi[kPer];
        int keep = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int i = tid * kPer + q;
          mi[q] = -1;
          if (i < cnt && cx[i] >= flt) { mx[q] = cx[i]; mi[q] = ci[i]; ++keep; }
        }
        int total = 0;
        int off = block_excl_scan_i32<NT>(keep, sh.red_i32, &total);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kPer; ++q)
          if (mi[q] >= 0) { cx[off] = mx[q]; ci[off] = mi[q]; ++off; }
        if (tid == 0) {
          sh.count = total;
          if (total > tcap / 2) sh.overflow = 1;  // ties hold the buffer
        }
        __syncthreads();
      }
    }
    __syncthreads();
    if (!sh.overflow) {
      // ---------------- exact warpers on the candidates -----------------
      const int cnt = sh.count;
      // Final scores after temperature.
      for (int i = tid; i < cnt; i += NT) cx[i] = (T == 1.0f) ? cx[i] : cx[i] / T;
      __syncthreads();
      const uint32_t tk = radix_kth_largest(
          [&](auto &&f) {
            for (int i = tid; i < cnt; i += NT) f(ordered_f32(cx[i]));
          },
          k_eff, rhist, sh);
      const float t_y = tk == 0u ? -INFINITY : unordered_f32(tk);
      // Keys of the kept ids, ordered.
      uint64_t *keys = reinterpret_cast<uint64_t *>(area + 8 * tcap);
      double *w = reinterpret_cast<double *>(area + 16 * tcap);
      if (tid == 0) sh.n_coll = 0;
      __syncthreads();
      for (int i = tid; i < cnt; i += NT)
        if (cx[i] >= t_y) {
          const int s = atomicAdd(&sh.n_coll, 1);
          keys[s] = sel_key(cx[i], (uint32_t)ci[i]);
        }
      __syncthreads();
      const int nk = sh.n_coll;
      if (nk == 0) {  // every id removed
        if (tid == 0) { sh.token = 0; sh.kcut = ~0ull; sh.t_y = INFINITY; }
        __syncthreads();
      } else {
      // Sort by ranks, using the candidate area as scratch.
      {
        uint64_t *tmpk = reinterpret_cast<uint64_t *>(area);  // cx/ci no longer needed
        for (int i = tid; i < nk; i += NT) {
          const uint64_t ki = keys[i];
          int r = 0;
          for (int j = 0; j < nk; ++j) r += keys[j] > ki;
          tmpk[r] = ki;
        }
        __syncthreads();
        for (int i = tid; i < nk; i += NT) keys[i] = tmpk[i];
        __syncthreads();
      }
      const double m = (double)key_score(keys[0]);
      for (int i = tid; i < nk; i += NT) w[i] = exp((double)key_score(keys[i]) - m);
      __syncthreads();
      if (tid == 0) {
        double W = 0.0;
        for (int j = 0; j < nk; ++j) W += w[j];
        int K = nk;
        if (use_top_p) {
          double run = 0.0;
          K = 0;
          for (int j = 0; j < nk; ++j) {
            if (run / W < p_top) K = j + 1;
            run += w[j];
          }
        }
        double Wp = 0.0;
        for (int j = 0; j < K; ++j) Wp += w[j];
        const double target = u * Wp;
        double C = 0.0;
        int pick = K - 1;
        for (int j = 0; j < K; ++j) {
          C += w[j];
          if (C > target) { pick = j; break; }
        }
        sh.token = (int)key_index(keys[pick]);
        sh.kcut = (use_top_p && K < nk) ? keys[K - 1] : 0ull;
        sh.t_y = t_y;
      }
      __syncthreads();
      }
      done = true;
    }
  }

  if (!done) {
    // ======================= full path ===================================
    // Row in registers when it fits (loaded now unless already in flight).
    if (RES > 0 && !full_first) {
#pragma unroll
      for (int i = 0; i < RES; ++i) {
        const int g = tid + i * NT;
        if (g < NG) reg[i] = load16(rowp + (int64_t)g * 16);
      }
    }
    const bool resident = RES > 0 && NG <= RES * NT;
    // Visit every element (dense + list): f(id, y, alive), y = final score
    // before top_k / top_p.
    auto visit_all = [&](auto &&f) {
      if (resident) {
#pragma unroll
        for (int i = 0; i < (RES > 0 ? RES : 1); ++i) {
          const int g = tid + i * NT;
          if (g < NG) {
            const uint32_t kb = chunk_bits<DT>(kbytes, g);
            const uint32_t sb = dense_pen ? chunk_bits<DT>(sbytes, g) : 0u;
#pragma unroll
            for (int j = 0; j < EPC; ++j) {
              float x = E::get(reg[i], j);
              if ((sb >> j) & 1u) x = penalize(x, rep);
              if (T != 1.0f) x = x / T;
              f(g * EPC + j, x, !((kb >> j) & 1u));
            }
          }
        }
      } else {
        stream_dense([&](int v, float x, bool alive) {
          if (T != 1.0f) x = x / T;
          f(v, x, alive);
        });
      }
      for (int i = tid; i < n_list; i += NT) {
        float x = list_val[i];
        if (T != 1.0f) x = x / T;
        f(list_id[i], x, true);
      }
    };

    // top_k that the candidate buffer could not hold: exact k-th largest by
    // a radix select over the whole row.
    float t_y = -INFINITY;
    if (k_eff > 0) {
      const uint32_t tk = radix_kth_largest(
          [&](auto &&f) {
            visit_all([&](int, float y, bool alive) {
              if (alive) f(ordered_f32(y));
            });
          },
          k_eff, rhist, sh);
      t_y = tk == 0u ? -INFINITY : unordered_f32(tk);
    }
    // Row max over the kept scores.
    float mx = -INFINITY;
    visit_all([&](int, float y, bool alive) {
      if (alive && y >= t_y) mx = fmaxf(mx, y);
    });
    mx = block_max_f32<NT>(mx, sh.red_f32);
    if (mx == -INFINITY) {
      if (tid == 0) {
        sh.token = 0;  // every id removed
        sh.kcut = ~0ull;
        sh.t_y = INFINITY;
      }
      __syncthreads();
    } else {
      // Mass histogram over bins of (max - y).
      const int nb = a.nb;
      const float bscale = (float)nb / kBinRange;
      float *hmass = reinterpret_cast<float *>(area);
      uint32_t *hcnt = reinterpret_cast<uint32_t *>(area + 4 * nb);
      uint64_t *ckey = reinterpret_cast<uint64_t *>(area + 8 * nb);
      float *cval = reinterpret_cast<float *>(area + 8 * nb + 8 * a.ccap);
      for (int i = tid; i < nb; i += NT) { hmass[i] = 0.0f; hcnt[i] = 0u; }
      __syncthreads();
      auto bin_of = [&](float y) {
        const float d = (mx - y) * bscale;
        return d < (float)(nb - 1) ? (int)d : nb - 1;
      };
      auto mass_of = [&](float y) { return __expf(y - mx); };
      visit_all([&](int, float y, bool alive) {
        if (alive && y >= t_y) {
          const float e = mass_of(y);
          const int b = bin_of(y);
          atomicAdd(&hmass[b], e);
          atomicAdd(&hcnt[b], 1u);
        }
      });
      __syncthreads();
      // Cumulative masses of the bins (binary64): S_b = mass of bins < b.
      double *cum = reinterpret_cast<double *>(area + 8 * nb + 12 * a.ccap);  // nb + 1 doubles
      if (tid < kWave) {
        double run = 0.0;
        const int per = (nb + kWave - 1) / kWave;
        double part = 0.0;
        for (int q = 0; q < per; ++q) {
          const int b = tid * per + q;
          if (b < nb) part += (double)hmass[b];
        }
        double incl = wave_incl_scan_f64(part);
        run = incl - part;
        for (int q = 0; q < per; ++q) {
          const int b = tid * per + q;
          if (b < nb) { cum[b] = run; run += (double)hmass[b]; }
        }
        if (tid == kWave - 1) cum[nb] = run;
      }
      __syncthreads();
      const double W = cum[nb];
      // Collect the elements of one bin as (key, mass), ordered; returns
      // the count, or -1 when the bin exceeds the collect capacity.
      auto collect_bin = [&](int bsel) -> int {
        if ((int)hcnt[bsel] > a.ccap) return -1;
        if (tid == 0) sh.n_coll = 0;
        __syncthreads();
        visit_all([&](int v, float y, bool alive) {
          if (alive && y >= t_y && bin_of(y) == bsel) {
            const int s = atomicAdd(&sh.n_coll, 1);
            if (s < a.ccap) { ckey[s] = sel_key(y, (uint32_t)v); cval[s] = mass_of(y); }
          }
        });
        __syncthreads();
        const int nc = min(sh.n_coll, a.ccap);
        // rank sort (keys distinct); scratch after cum[]
        uint64_t *tk2 = reinterpret_cast<uint64_t *>(area + 8 * nb + 12 * a.ccap + 8 * (nb + 1));
        float *tv2 = reinterpret_cast<float *>(tk2 + a.ccap);
        rank_sort_desc<float>(ckey, cval, nc, tk2, tv2);
        return nc;
      };
      // Mass of the elements of bin bsel whose key is > q (ge = false) or
      // >= q (ge = true), for the bisection on oversized bins.
      auto bin_mass_above = [&](int bsel, uint64_t q, bool ge, uint64_t kmin) -> double {
        double s = 0.0;
        visit_all([&](int v, float y, bool alive) {
          if (alive && y >= t_y && bin_of(y) == bsel) {
            const uint64_t kk = sel_key(y, (uint32_t)v);
            if (kk >= kmin && (ge ? kk >= q : kk > q)) s += (double)mass_of(y);
          }
        });
        return block_sum_f64<NT>(s, sh.red_f64);
      };

      // ---- top_p cutoff ----
      uint64_t kcut = 0ull;   // kept iff key >= kcut
      double Wp = W;          // kept mass
      int bp = nb;            // bin of the cutoff (nb: none)
      if (use_top_p) {
        const double pw = p_top * W;
        // smallest b with cum[b+1] >= p W
        if (tid == 0) {
          int lo = 0, hi = nb - 1, ans = nb;
          while (lo <= hi) {
            const int mid = (lo + hi) / 2;
            if (cum[mid + 1] >= pw) { ans = mid; hi = mid - 1; } else lo = mid + 1;
          }
          sh.bin_p = ans;
        }
        __syncthreads();
        bp = sh.bin_p;
        if (bp < nb) {
          const double Sb = cum[bp];
          const int nc = collect_bin(bp);
          if (nc >= 0) {
            if (tid == 0) {
              double run = 0.0;
              int K = nc;
              for (int j = 0; j < nc; ++j) {
                if (Sb + run >= pw) { K = j; break; }
                run += (double)cval[j];
              }
              // Kept: every element of earlier bins, the first K of this bin.
              if (K == 0) {
                // The boundary sits on the bin edge: keep bins < bp.
                sh.kcut = ckey[0] + 1ull;
                sh.wprime = Sb;
              } else {
                sh.kcut = ckey[K - 1];
                double kept = 0.0;
                for (int j = 0; j < K; ++j) kept += (double)cval[j];
                sh.wprime = Sb + kept;
              }
            }
            __syncthreads();
          } else {
            // Bisection over keys: q* = min{q : Sb + mass(key > q) < pW}.
            uint64_t lo = 0ull, hi = ~0ull;
            while (hi - lo > 1ull) {
              const uint64_t mid = lo + (hi - lo) / 2;
              const double g = Sb + bin_mass_above(bp, mid, false, 0ull);
              if (g < pw) hi = mid; else lo = mid;
            }
            const double wk = bin_mass_above(bp, hi, true, 0ull);
            if (tid == 0) { sh.kcut = hi; sh.wprime = Sb + wk; }
            __syncthreads();
          }
          kcut = sh.kcut;
          Wp = sh.wprime;
        }
      }
      // ---- inverse-CDF draw ----
      const double target = u * Wp;
      // smallest b with (mass of kept elements in bins <= b) > target
      if (tid == 0) {
        int lo = 0, hi = min(bp, nb - 1), ans = -1;
        while (lo <= hi) {
          const int mid = (lo + hi) / 2;
          const double c = (mid < bp) ? cum[mid + 1] : Wp;
          if (c > target) { ans = mid; hi = mid - 1; } else lo = mid + 1;
        }
        if (ans < 0) ans = min(bp, nb - 1);  // rounding: the last kept bin
        sh.bin_u = ans;
      }
      __syncthreads();
      const int bu = sh.bin_u;
      const double Su = cum[bu];
      const int nc = collect_bin(bu);
      if (nc >= 0) {
        if (tid == 0) {
          double C = Su;
          int pick = -1, last = -1;
          for (int j = 0; j < nc; ++j) {
            if (ckey[j] < kcut) break;
            last = j;
            C += (double)cval[j];
            if (C > target) { pick = j; break; }
          }
          if (pick < 0) pick = last;
          sh.found = pick;
          sh.token = pick >= 0 ? (int)key_index(ckey[pick]) : -1;
        }
        __syncthreads();
      } else {
        if (tid == 0) sh.found = -1;
        __syncthreads();
      }
      if (sh.found < 0) {
        // Bisection: the token key is max{q : Su + mass(key >= q, kept) > target}.
        uint64_t lo = kcut, hi = ~0ull;
        if (Su + bin_mass_above(bu, lo, true, kcut) > target) {
          while (hi - lo > 1ull) {
            const uint64_t mid = lo + (hi - lo) / 2;
            if (Su + bin_mass_above(bu, mid, true, kcut) > target) lo = mid; else hi = mid;
          }
        } else {
          // rounding: the smallest kept key of the bin
          uint64_t best = 0ull;
          visit_all([&](int v, float y, bool alive) {
            if (alive && y >= t_y && bin_of(y) == bu) {
              const uint64_t kk = sel_key(y, (uint32_t)v);
              if (kk >= kcut) best = max(best, ~kk);
            }
          });
          best = block_max_u64<NT>(best, sh.red_u64);
          lo = ~best;
        }
        if (tid == 0) sh.token = (int)key_index(lo);
        __syncthreads();
      }
      if (tid == 0) {
        sh.kcut = kcut;
        sh.t_y = t_y;
      }
      __syncthreads();
    }
  }

  if (tid == 0) a.out_tokens[row] = sh.token;
  if (outp) {
    // Final scores: the score after temperature when kept, else -inf.
    const uint64_t kcut = sh.kcut;
    const float t_y = sh.t_y;
    stream_dense([&](int v, float x, bool alive) {
      const float y = (T != 1.0f) ? x / T : x;
      outp[v] = (alive && y >= t_y && sel_key(y, (uint32_t)v) >= kcut) ? y : -INFINITY;
    });
    for (int v = Vvec + tid; v < V; v += NT) outp[v] = -INFINITY;
    __syncthreads();
    for (int i = tid; i < n_list; i += NT) {
      const float y = (T != 1.0f) ? list_val[i] / T : list_val[i];
      outp[list_id[i]] = (y >= t_y && sel_key(y, (uint32_t)list_id[i]) >= kcut) ? y : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
template <int DT, int RES>
static hipError_t launch_select_t(const SelectArgs &a, size_t lds, hipStream_t s) {
  static bool attr_set = false;  // benign race: every writer stores the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_select<DT, RES>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kSelectMaxDynLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_select<DT, RES>), dim3(a.B), dim3(NT), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs &a, int res, size_t lds, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.dtype == 1) {
    switch (res) {
      case 4: return launch_select_t<1, 4>(a, lds, s);
      case 8: return launch_select_t<1, 8>(a, lds, s);
      case 16: return launch_select_t<1, 16>(a, lds, s);
      default: return launch_select_t<1, 0>(a, lds, s);
    }
  }
  switch (res) {
    case 4: return launch_select_t<0, 4>(a, lds, s);
    case 8: return launch_select_t<0, 8>(a, lds, s);
    case 16: return launch_select_t<0, 16>(a, lds, s);
    default: return launch_select_t<0, 0>(a, lds, s);
  }
}

}  // namespace tsel
