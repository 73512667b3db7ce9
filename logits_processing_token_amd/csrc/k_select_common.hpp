// k_select_common.hpp -- pieces shared by the selection kernels (k_greedy,
// k_topk, k_full): element access, on-chip layout, the row prologue, the
// staging of the history and masks, the row stream and the radix select.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsel_device.hpp"
#include "tsel_internal.hpp"

namespace tsel {

constexpr int NT = kSelectThreads;
constexpr int NW = NT / kWave;
constexpr int U = 4;                 // 16-byte chunks per lane per batch when streaming
                                     // (two batches: one consumed, one in flight)
constexpr uint32_t kNoDigit = 0xFFFFFFFFu;
constexpr int kPending = -2;         // token marker: row left for k_full
constexpr float kLog2e = 1.4426950408889634f;

// The log-probability of a row without a token, or whose scores are all
// -inf: the quiet NaN with sign bit 0.
__device__ __forceinline__ float lp_none() { return __uint_as_float(0x7FC00000u); }

// Running (max, sum of exp(x - max)) of one thread's finite scores in
// binary64; the sum is rescaled when the maximum moves.
struct LseAcc {
  double m = -INFINITY;
  double s = 0.0;
  __device__ __forceinline__ void add(float xf) {
    const double x = (double)xf;
    if (!(x > -INFINITY)) return;
    if (x > m) {
      s = s * exp(m - x) + 1.0;  // (exp(-inf) = 0 on the first score)
      m = x;
    } else {
      s += exp(x - m);
    }
  }
};

// The largest finite score M over the workgroup (-inf if none) and S = sum
// exp(x - M), joining every thread's pair at M.  Every thread calls.
template <int NT_>
__device__ __forceinline__ void lse_join(const LseAcc &acc, float *rmax, double *rsum,
                                         float *M_out, double *S_out) {
  const float M = block_max_f32<NT_>((float)acc.m, rmax);
  double part = 0.0;
  if (acc.m > -INFINITY) part = acc.s * exp(acc.m - (double)M);
  *S_out = block_sum_f64<NT_>(part, rsum);
  *M_out = M;
}

template <int DT>
struct Elem;
template <>
struct Elem<0> {  // binary32
  static constexpr int EPC = 4;
  static constexpr uint32_t kNegInf = 0xFF800000u;
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
  static constexpr uint32_t kNegInf = 0xFF80FF80u;
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
  int n_list;
  int dense_pen;
  int count;
  int overflow;
  uint32_t digit;
  int krem;
  float tau_x;
  int token;
  uint64_t kcut;
  float t_y;
  int bin_p, bin_hi;
  int n_coll;
  double wprime;
  double sbase;
  float ylo, yhi;
  int found;
};

// On-chip regions of one workgroup (offsets from SelectArgs).
struct Lds {
  uint32_t *kmask, *smask;
  int32_t *list_id;
  float *list_val;
  uint4 *lut;
  uint32_t *rhist;
  unsigned char *area;
};

__device__ __forceinline__ Lds carve(const SelectArgs &a, unsigned char *smem) {
  Lds s;
  s.kmask = reinterpret_cast<uint32_t *>(smem + a.off_kmask);
  s.smask = reinterpret_cast<uint32_t *>(smem + a.off_smask);
  s.list_id = reinterpret_cast<int32_t *>(smem + a.off_list_id);
  s.list_val = reinterpret_cast<float *>(smem + a.off_list_val);
  s.lut = reinterpret_cast<uint4 *>(smem + a.off_lut);
  s.rhist = reinterpret_cast<uint32_t *>(smem + a.off_rhist);
  s.area = smem + a.off_area;
  return s;
}

__device__ __forceinline__ uint4 load16(const char *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

// Mask bits of chunk g: bit j covers element g * EPC + j.
template <int DT>
__device__ __forceinline__ uint32_t chunk_bits(const uint32_t *m, int g) {
  const uint8_t *b = reinterpret_cast<const uint8_t *>(m);
  if (DT == 1) return b[g];
  return (b[g >> 1] >> ((g & 1) * 4)) & 0xFu;
}

__device__ __forceinline__ bool bit_of(const uint32_t *m, int v) {
  return (m[v >> 5] >> (v & 31)) & 1u;
}

// Killed elements of a chunk become -inf in place: the kill bits index a
// table of 16-byte masks, one bit-field insert per 32-bit word.
template <int DT>
__device__ __forceinline__ uint4 kill_chunk(uint4 c, int g, const Lds &s) {
  const uint4 m = s.lut[chunk_bits<DT>(s.kmask, g)];
  const uint32_t ninf = Elem<DT>::kNegInf;
  c.x = (m.x & ninf) | (~m.x & c.x);
  c.y = (m.y & ninf) | (~m.y & c.y);
  c.z = (m.z & ninf) | (~m.z & c.z);
  c.w = (m.w & ninf) | (~m.w & c.w);
  return c;
}

// Smallest binary32 x with RN(x / T) >= RN(tau / T): the pre-temperature
// threshold admitting every score the temperature maps onto tau's value
// (division by T > 0 is monotone but can merge neighbours).
__device__ inline float pre_temperature_floor(float tau, float T) {
  if (T == 1.0f || tau == -INFINITY) return tau;
  const float t = tau / T;
  uint32_t hi = ordered_f32(tau), lo = 0;
  while (hi - lo > 1) {
    const uint32_t mid = lo + (hi - lo) / 2;
    if (unordered_f32(mid) / T >= t) hi = mid; else lo = mid;
  }
  return unordered_f32(hi);
}

// k-th largest of a multiset of ordered keys by an LDS radix select over four
// 8-bit digits; visit(f) calls f(key) once per element (all threads
// together).  Returns 0 when there are fewer than k elements.
template <class Visit>
__device__ __forceinline__ uint32_t radix_kth_largest(Visit &&visit, int k, uint32_t *hist, RowShared &sh) {
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
      const uint32_t c0 = hist[255 - 4 * l], c1 = hist[254 - 4 * l], c2 = hist[253 - 4 * l],
                     c3 = hist[252 - 4 * l];
      const int s = (int)(c0 + c1 + c2 + c3);
      const int incl = wave_incl_scan_i32(s);
      const int excl = incl - s;
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

// A lower bound of the k-th largest of the values that visit(f) passes to
// f (every thread calls; values above -inf): the values are counted into
// nbins (NT, 2 NT or 4 NT) equal-width bins spanning their minimum to
// maximum (spread out, so the LDS adds rarely meet on one word), and the
// bound is the lower edge of the bin one below the one holding the k-th
// largest (a bin of slack for the rounding of the bin arithmetic).  -inf
// when there are fewer than k values.  hist: nbins words.
template <class Visit>
__device__ __forceinline__ float kth_lower_bound(Visit &&visit, int k, uint32_t *hist, int nbins,
                                                 RowShared &sh) {
  const int tid = threadIdx.x;
  float lmax = -INFINITY, lmin = INFINITY;
  int lcnt = 0;
  visit([&](float x) {
    lmax = fmaxf(lmax, x);
    lmin = fminf(lmin, x);
    ++lcnt;
  });
  for (int i = tid; i < nbins; i += NT) hist[i] = 0u;
  // the maximum, minimum and count in one exchange (one barrier; the scan
  // below passes a barrier before it writes these slots again)
  {
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    const float wmx = wave_max_f32_uni(lmax), wmn = -wave_max_f32_uni(-lmin);
    const int wc = __builtin_amdgcn_readlane(wave_incl_scan_i32(lcnt), kWave - 1);
    if (lane == 0) {
      sh.red_f32[wid] = wmx;
      sh.red_u64[wid] = __float_as_uint(wmn);
      sh.red_i32[wid] = wc;
    }
  }
  __syncthreads();
  float mx = -INFINITY, mn = INFINITY;
  int n = 0;
#pragma unroll
  for (int q = 0; q < NT / kWave; ++q) {
    mx = fmaxf(mx, sh.red_f32[q]);
    mn = fminf(mn, __uint_as_float((uint32_t)sh.red_u64[q]));
    n += sh.red_i32[q];
  }
  if (n < k || k < 1) return -INFINITY;
  if (!(mx > mn)) return mn;
  const float scale = (float)(nbins - 1) / (mx - mn);  // (0 if the span overflows)
  visit([&](float x) {
    const int b = min(max((int)((x - mn) * scale), 0), nbins - 1);
    atomicAdd(&hist[b], 1u);
  });
  __syncthreads();
  // thread t holds bins nbins - 1 - bpt t downwards (from the top); the
  // counts above its bins by an exclusive scan over threads
  const int bpt = nbins / NT;
  const int top = nbins - 1 - bpt * tid;
  uint32_t c[4];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = q < bpt ? hist[top - q] : 0u;
    mine += (int)c[q];
  }
  int total;
  int above = block_excl_scan_i32<NT>(mine, sh.red_i32, &total);
  if (tid == 0) sh.found = 0;
  __syncthreads();
  if (above < k && k <= above + mine) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      above += (int)c[q];
      if (above >= k) {
        sh.found = top - q;
        break;
      }
    }
  }
  __syncthreads();
  const int b = sh.found;
  return b <= 1 || scale == 0.0f ? mn : mn + (float)(b - 1) / scale;
}

// ---------------------------------------------------------------------------
// Row prologue: padding rows (no token) and forced rows (forced_bos at one
// token, forced_eos at max_length - 1; the later processor wins; a forced id
// that suppress / begin-suppress then removes leaves an all-removed row, id
// 0).  Returns true when the row is finished.
struct RowInfo {
  int L, P, M, new_tokens;
  bool begin_active;
};

// The row's lengths (history, prompt, max_length), read on their own so
// that a kernel can start these loads before any other.
__device__ __forceinline__ void row_lens(const SelectArgs &a, int row, RowInfo &ri) {
  ri.L = a.lens[row];
  ri.P = a.lens[a.B + row];
  ri.M = a.lens[2 * a.B + row];
}

// The same through vector loads, which are counted in issue order with the
// row's own, so that they are not pushed behind them; the values end in
// scalar registers.
__device__ __forceinline__ void row_lens_vector(const SelectArgs &a, int row, RowInfo &ri) {
  ri.L = __builtin_amdgcn_readfirstlane(__builtin_nontemporal_load(a.lens + row));
  ri.P = __builtin_amdgcn_readfirstlane(__builtin_nontemporal_load(a.lens + a.B + row));
  ri.M = __builtin_amdgcn_readfirstlane(__builtin_nontemporal_load(a.lens + 2 * a.B + row));
}

// The prologue once row_lens has run.
__device__ __forceinline__ bool row_prologue_after_lens(const SelectArgs &a, int row, RowInfo &ri) {
  const int tid = threadIdx.x;
  const int V = a.V;
  ri.new_tokens = ri.L - ri.P;
  ri.begin_active =
      a.begin_mask != nullptr && ri.new_tokens == ((a.forced_bos >= 0 && ri.P == 1) ? 1 : 0);
  float *outp = a.out_processed ? a.out_processed + (int64_t)row * V : nullptr;
  if (ri.L <= 0) {
    if (tid == 0) {
      a.out_tokens[row] = -1;
      if (a.out_logprobs) a.out_logprobs[row] = lp_none();
    }
    if (outp)
      for (int v = tid; v < V; v += NT) outp[v] = -INFINITY;
    return true;
  }
  int forced = -1;
  if (a.forced_bos >= 0 && ri.L == 1) forced = a.forced_bos;
  if (a.forced_eos >= 0 && ri.L == ri.M - 1) forced = a.forced_eos;
  if (forced >= 0) {
    bool alive = forced < V;
    if (alive && a.sup_mask && bit_of(a.sup_mask, forced)) alive = false;
    if (alive && ri.begin_active && bit_of(a.begin_mask, forced)) alive = false;
    if (tid == 0) {
      a.out_tokens[row] = alive ? forced : 0;
      // (the lone score 0 has log-probability 0)
      if (a.out_logprobs) a.out_logprobs[row] = alive ? 0.0f : lp_none();
    }
    if (outp)
      for (int v = tid; v < V; v += NT) outp[v] = (alive && v == forced) ? 0.0f : -INFINITY;
    return true;
  }
  return false;
}

__device__ __forceinline__ bool row_prologue(const SelectArgs &a, int row, RowInfo &ri) {
  row_lens(a, row, ri);
  return row_prologue_after_lens(a, row, ri);
}

// Staging of one row (see the file comment).  Leaves in LDS: the kill mask
// (seen ids included unless dense_pen), the seen mask, the list of
// (id, penalized logit) and the kill-mask table.
// prefer_dense: the caller streams the row anyway, so the penalty may be
// applied in the stream (from the seen mask) rather than to gathered scores
// whenever the seen ids would touch a large share of the row's cache lines
// (a gather pulls a whole line for one score).
template <int DT>
__device__ __forceinline__ void stage_row(const SelectArgs &a, int row, const RowInfo &ri, const Lds &s,
                          RowShared &sh, bool prefer_dense = true) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  const int tid = threadIdx.x;
  const int V = a.V;
  const int NG = V / EPC;
  const int Vvec = NG * EPC;
  const int L = ri.L;
  const int mw = a.mw;
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  for (int w = tid; w < mw; w += NT) {
    s.kmask[w] = 0u;
    s.smask[w] = 0u;
  }
  // table: kill bits of a chunk -> per-word masks of its killed elements
  if (DT == 1) {
    if (tid < 256) {
      const uint32_t v = (uint32_t)tid;
      uint32_t m[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        m[j] = (((v >> (2 * j)) & 1u) ? 0x0000FFFFu : 0u) |
               (((v >> (2 * j + 1)) & 1u) ? 0xFFFF0000u : 0u);
      s.lut[tid] = make_uint4(m[0], m[1], m[2], m[3]);
    }
  } else {
    if (tid < 16) {
      const uint32_t v = (uint32_t)tid;
      s.lut[tid] = make_uint4((v & 1u) ? ~0u : 0u, (v & 2u) ? ~0u : 0u, (v & 4u) ? ~0u : 0u,
                              (v & 8u) ? ~0u : 0u);
    }
  }
  __syncthreads();
  const int32_t *h = a.hist + (int64_t)row * a.hist_stride;
  // Seen ids and n-gram windows in batches of kHB ids per thread, every
  // load of a batch in flight at once.  Window i bans its last id when its
  // first n-1 ids equal the last n-1 ids of the history ("Lengths",
  // no_repeat_ngram_size); its first id, already loaded, rules most windows
  // out.
  constexpr int kHB = 8;
  const int n = a.ngram;
  const bool ngram = n > 0 && L >= n;
  const int32_t *tail = h + (L - n + 1);
  const int tail0 = ngram && n > 1 ? tail[0] : 0;
  for (int base = 0; base < L; base += NT * kHB) {
    int hv[kHB];
#pragma unroll
    for (int k = 0; k < kHB; ++k) {
      const int i = base + k * NT + tid;
      hv[k] = i < L ? h[i] : -1;
    }
#pragma unroll
    for (int k = 0; k < kHB; ++k) {
      const int i = base + k * NT + tid;
      const int v = hv[k];
      if (v >= 0 && v < V) atomicOr(&s.smask[v >> 5], 1u << (v & 31));
      if (ngram && i + n <= L && (n == 1 || v == tail0)) {
        bool match = true;
        for (int j = 1; j < n - 1; ++j)
          if (h[i + j] != tail[j]) { match = false; break; }
        const int t = h[i + n - 1];
        if (match && t >= 0 && t < V) atomicOr(&s.kmask[t >> 5], 1u << (t & 31));
      }
    }
  }
  const bool minlen_active = a.min_new > 0 ? (ri.new_tokens < a.min_new)
                                           : (a.min_length > 0 && L < a.min_length);
  if (minlen_active && tid < a.n_eos) {
    const int e = a.eos[tid];
    if (e >= 0 && e < V) atomicOr(&s.kmask[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  // Fold the static masks in; count the seen ids that stay alive.
  const int wpt = (mw + NT - 1) / NT;  // contiguous words per thread
  int my_cnt = 0;
  for (int q = 0; q < wpt; ++q) {
    const int w = tid * wpt + q;
    if (w < mw) {
      uint32_t k = s.kmask[w];
      if (a.bad_mask) k |= a.bad_mask[w];
      if (a.sup_mask) k |= a.sup_mask[w];
      if (ri.begin_active) k |= a.begin_mask[w];
      s.kmask[w] = k;
      my_cnt += __popc(s.smask[w] & ~k);
    }
  }
  int n_seen = 0;
  const int my_off = block_excl_scan_i32<NT>(my_cnt, sh.red_i32, &n_seen);
  const bool dense_pen = n_seen > a.lcap - 8 || (prefer_dense && (int64_t)n_seen * 64 > NG);
  if (!dense_pen) {
    int o = my_off;
    for (int q = 0; q < wpt; ++q) {
      const int w = tid * wpt + q;
      if (w < mw) {
        uint32_t bits = s.smask[w] & ~s.kmask[w];
        while (bits) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1;
          s.list_id[o++] = w * 32 + b;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int o = dense_pen ? 0 : n_seen;
    for (int v = Vvec; v < V; ++v) {
      const bool killed = bit_of(s.kmask, v) || (!dense_pen && bit_of(s.smask, v));
      if (!killed) s.list_id[o++] = v;
    }
    sh.n_list = o;
    sh.dense_pen = dense_pen ? 1 : 0;
  }
  __syncthreads();
  if (!dense_pen)  // the stream kills seen ids; the list carries them
    for (int w = tid; w < mw; w += NT) s.kmask[w] |= s.smask[w];
  const int n_list = sh.n_list;
  for (int base = 0; base < n_list; base += NT * kHB) {  // (gathers in flight together)
    float xv[kHB];
#pragma unroll
    for (int k = 0; k < kHB; ++k) {
      const int i = base + k * NT + tid;
      xv[k] = i < n_list ? E::load1(rowp, s.list_id[i]) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kHB; ++k) {
      const int i = base + k * NT + tid;
      if (i < n_list) {
        const int v = s.list_id[i];
        s.list_val[i] = bit_of(s.smask, v) ? penalize(xv[k], a.rep) : xv[k];
      }
    }
  }
  __syncthreads();
}

// Visit the dense elements of this lane in increasing id order, streaming
// from global memory: f(id, x) with x after kill (-inf) and, in dense_pen
// mode, after the penalty.
template <int DT, class F>
__device__ __forceinline__ void stream_row(const SelectArgs &a, const char *rowp, const Lds &s,
                                           bool dense_pen, F &&f) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  const int NG = a.V / EPC;
  // two batches of U chunks: the next batch's loads fly while this one is
  // consumed
  uint4 c[U], nx[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = threadIdx.x + u * NT;
    if (g < NG) c[u] = load16(rowp + (int64_t)g * 16);
  }
  for (int g0 = threadIdx.x; g0 < NG; g0 += NT * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + NT * U + u * NT;
      if (g < NG) nx[u] = load16(rowp + (int64_t)g * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * NT;
      if (g < NG) {
        const uint4 ck = kill_chunk<DT>(c[u], g, s);
        const uint32_t sb = dense_pen ? chunk_bits<DT>(s.smask, g) : 0u;
#pragma unroll
        for (int j = 0; j < EPC; ++j) {
          float x = E::get(ck, j);
          if ((sb >> j) & 1u) x = penalize(x, a.rep);
          f(g * EPC + j, x);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) c[u] = nx[u];
  }
}

// Final processed scores of a sampled row: the score after temperature when
// kept (>= the top_k threshold t_y and selection key >= kcut), else -inf.
template <int DT>
__device__ __forceinline__ void write_processed(const SelectArgs &a, int row, const Lds &s, RowShared &sh,
                                float t_y, uint64_t kcut) {
  constexpr int EPC = Elem<DT>::EPC;
  const int tid = threadIdx.x, V = a.V;
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  float *outp = a.out_processed + (int64_t)row * V;
  const float T = a.temperature;
  stream_row<DT>(a, rowp, s, sh.dense_pen != 0, [&](int v, float x) {
    const float y = (T != 1.0f) ? x / T : x;
    outp[v] = (y > -INFINITY && y >= t_y && sel_key(y, (uint32_t)v) >= kcut) ? y : -INFINITY;
  });
  for (int v = (V / EPC) * EPC + tid; v < V; v += NT) outp[v] = -INFINITY;
  __syncthreads();
  const int n_list = sh.n_list;
  for (int i = tid; i < n_list; i += NT) {
    const float y = (T != 1.0f) ? s.list_val[i] / T : s.list_val[i];
    outp[s.list_id[i]] =
        (y >= t_y && sel_key(y, (uint32_t)s.list_id[i]) >= kcut) ? y : -INFINITY;
  }
}

}  // namespace tsel
