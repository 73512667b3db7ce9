// k_res_common.hpp -- pieces shared by the resident-row sampling kernels
// (k_res: mass bins, any element type; k_vres: one bin per bf16 value): the
// small loads and the LDS staging that run while the row is in flight, the
// walk of a bin whose dense elements tie, and the final-score writer.
//
// Sources: "Transmuter.Generation (transmuter v2.0.0)", module doc (the
// processors in order: repetition penalty over the seen ids, no-repeat
// n-grams, bad words, minimum length, suppression; then the top_p warper and
// the inverse-CDF draw of a caller uniform over the kept ids in (score desc,
// id asc) order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k_mass.hpp"

namespace tsel {
namespace res {

constexpr int kPipe = 8;  // 16-byte chunks in flight per lane
constexpr int kHpt = 4;   // history ids per thread held in registers
constexpr int kMpt = 4;   // kill-mask words per thread: V <= 32 * kMpt * NT

enum : int { kFail = -1, kInd = 0, kGroup = 1, kCollect = 2, kNone = 3 };

// Order of a bin whose dense elements hold one value: individual elements
// (seen ids, or anything else listed one by one) above the value, the tie
// group (dense elements of the value and individuals equal to it, in id
// order), individuals below the value.  Positions are linear in that order.
struct BinView {
  int single;        // the bin's dense elements all hold one value
  float v;           // that value
  float e;           // its mass
  int n_ind;         // individuals of the bin not equal to v (sorted, okey / oval)
  int n_above;       // of them, above v
  int n_group;       // members of the tie group
};

struct WalkResult {
  int kind;          // kInd, kGroup or kFail
  uint64_t key;      // kInd: the element's key
  int rank;          // kGroup: 0-based rank in the group
  int pos;           // linear position in the bin
  double acc;        // cut: mass through the last kept element
};

// Walk of a single-valued bin (one thread).  cut: the last element kept by
// top_p (the first element whose mass before it is >= goal and everything
// after it are removed); draw: the first element whose mass through it
// exceeds goal, among positions <= pos_lim.
__device__ inline WalkResult single_walk(bool cut, double start, double goal, const BinView &bv,
                                         const uint64_t *okey, const float *oval, int pos_lim) {
  WalkResult r;
  r.kind = kFail;
  r.key = 0ull;
  r.rank = -1;
  r.pos = -1;
  r.acc = 0.0;
  double A = start;
  const double e = (double)bv.e;
  const int na = bv.n_above, ni = bv.n_ind, ng = bv.n_group;
  if (cut) {
    for (int q = 0; q < na; ++q) {
      if (A >= goal) { r.acc = A; return r; }
      A += (double)oval[q];
      r.kind = kInd; r.key = okey[q]; r.pos = q;
    }
    if (ng > 0) {
      if (A >= goal) { r.acc = A; return r; }
      // first member j with A + j e >= goal; j >= 1 since A < goal
      const double q = (goal - A) / e;  // finite and <= ng + a rounding in any bin
      long long j = q < (double)ng ? (long long)ceil(q) : (long long)ng;
      if (j < 1) j = 1;
      while (j > 1 && A + (double)(j - 1) * e >= goal) --j;
      while (j < ng && A + (double)j * e < goal) ++j;
      if (j < ng) {
        r.kind = kGroup; r.rank = (int)j - 1; r.pos = na + (int)j - 1;
        r.acc = A + (double)j * e;
        return r;
      }
      A += (double)ng * e;
      r.kind = kGroup; r.rank = ng - 1; r.pos = na + ng - 1;
    }
    for (int q = na; q < ni; ++q) {
      if (A >= goal) { r.acc = A; return r; }
      A += (double)oval[q];
      r.kind = kInd; r.key = okey[q]; r.pos = ng + q;
    }
    r.acc = A;
    return r;
  }
  // draw
  WalkResult last;
  last.kind = kFail;
  last.key = 0ull;
  last.rank = -1;
  last.pos = -1;
  last.acc = 0.0;
  for (int q = 0; q < na && q <= pos_lim; ++q) {
    A += (double)oval[q];
    last.kind = kInd; last.key = okey[q]; last.pos = q;
    if (A > goal) return last;
  }
  const int n_eff = pos_lim - na >= ng ? ng : pos_lim - na + 1;  // (no overflow at INT_MAX)
  if (n_eff > 0) {
    const double q = (goal - A) / e;
    long long j = q < (double)n_eff ? (long long)floor(q) : (long long)(n_eff - 1);
    if (j < 0) j = 0;
    while (j > 0 && A + (double)j * e > goal) --j;
    while (j < n_eff - 1 && A + (double)(j + 1) * e <= goal) ++j;
    last.kind = kGroup; last.rank = (int)j; last.pos = na + (int)j;
    if (A + (double)(j + 1) * e > goal) return last;
    A += (double)n_eff * e;
    last.rank = n_eff - 1; last.pos = na + n_eff - 1;
  }
  for (int q = na; q < ni && ng + q <= pos_lim; ++q) {
    A += (double)oval[q];
    last.kind = kInd; last.key = okey[q]; last.pos = ng + q;
    if (A > goal) return last;
  }
  return last;  // rounding at the end: the last element within the limit
}

// Slot on the list of seen id v (alive seen ids are listed in id order;
// woff[w] is the list offset of mask word w).
__device__ __forceinline__ int list_slot(int v, const uint32_t *amask, const uint16_t *woff) {
  const int w = v >> 5;
  return (int)woff[w] + __popc(amask[w] & ((1u << (v & 31)) - 1u));
}

// Hides a chunk's value from the optimizer, so that the elements unpacked
// from it are not computed early and kept live (which spills).
__device__ __forceinline__ uint4 launder(uint4 c) {
  asm volatile("" : "+v"(c.x), "+v"(c.y), "+v"(c.z), "+v"(c.w));
  return c;
}

// Element j of a chunk as its raw word bits, for building the tail chunk.
template <int DT>
__device__ __forceinline__ void put_elem(uint32_t *w, int j, uint32_t bits) {
  if (DT == 1) {
    const int q = j >> 1;
    w[q] = (j & 1) ? ((w[q] & 0x0000FFFFu) | (bits << 16)) : ((w[q] & 0xFFFF0000u) | bits);
  } else {
    w[j] = bits;
  }
}

// Final scores of a sampled row (kept: score >= t_y and key >= kcut, else
// -inf), one element per thread and step from memory; seen ids take their
// penalized score from the list.
template <int DT>
__device__ __forceinline__ void res_processed(const SelectArgs &a, int row, const Lds &s,
                                              float t_y, uint64_t kcut, int n_list) {
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  float *outp = a.out_processed + (int64_t)row * a.V;
  visit_plain<DT>(a, rowp, s, [&](int v, float y) {
    outp[v] = (y > -INFINITY && y >= t_y && sel_key(y, (uint32_t)v) >= kcut) ? y : -INFINITY;
  });
  for (int v = threadIdx.x; v < a.V; v += NT)
    if (bit_of(s.kmask, v)) outp[v] = -INFINITY;
  __syncthreads();
  for (int i = threadIdx.x; i < n_list; i += NT) {
    const float y = s.list_val[i];
    outp[s.list_id[i]] = (y >= t_y && sel_key(y, (uint32_t)s.list_id[i]) >= kcut) ? y : -INFINITY;
  }
}

// The small loads of a resident row, issued at the very start together with
// the row's own (none of them waits for the row's lengths): history ids
// (up to the history stride; entries past the row's length are ignored
// later), kill-mask words and the row tail (V % EPC ids after the last whole
// chunk, as one more chunk).  Every load is unconditional and in bounds -- an
// absent mask or history reads word 0 of the lengths and discards it, every
// lane loads the same few tail elements -- so that no branch splits the loads
// and the row's chunks can later be waited for one at a time.
struct Early {
  int hreg[kHpt];
  uint32_t km[kMpt];    // bad words | suppress
  uint32_t kbeg[kMpt];  // begin-suppress, for rows where it applies
  uint32_t tw[4];
};

template <int DT>
__device__ __forceinline__ void early_loads(const SelectArgs &a, int row, const char *rowp,
                                            Early &e) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  const int tid = threadIdx.x, V = a.V, mw = a.mw;
  const int NG = V / EPC;
  const uint32_t *lens_u = reinterpret_cast<const uint32_t *>(a.lens);
  const int32_t *hp = a.hist_stride > 0 ? a.hist + (int64_t)row * a.hist_stride : a.lens;
  const int hlast = max(a.hist_stride, 1) - 1;
#pragma unroll
  for (int k = 0; k < kHpt; ++k) e.hreg[k] = hp[min(tid + k * NT, hlast)];
  const uint32_t *m0p = a.bad_mask ? a.bad_mask : lens_u;
  const uint32_t *m1p = a.sup_mask ? a.sup_mask : lens_u;
  const uint32_t *m2p = a.begin_mask ? a.begin_mask : lens_u;
  const uint32_t m0k = a.bad_mask ? ~0u : 0u, m1k = a.sup_mask ? ~0u : 0u;
  const uint32_t m2k = a.begin_mask ? ~0u : 0u;
#pragma unroll
  for (int q = 0; q < kMpt; ++q) {
    const int w = min(tid * kMpt + q, mw - 1);
    e.km[q] = (m0p[m0k ? w : 0] & m0k) | (m1p[m1k ? w : 0] & m1k);
    e.kbeg[q] = m2p[m2k ? w : 0] & m2k;
  }
  const int tail_n = V - NG * EPC;
#pragma unroll
  for (int q = 0; q < 4; ++q) e.tw[q] = E::kNegInf;
#pragma unroll
  for (int j = 0; j < EPC - 1; ++j) {
    const int v = min(NG * EPC + j, V - 1);
    const uint32_t bits = DT == 1 ? (uint32_t)reinterpret_cast<const uint16_t *>(rowp)[v]
                                  : reinterpret_cast<const uint32_t *>(rowp)[v];
    const uint32_t ninf = DT == 1 ? 0xFF80u : 0xFF800000u;
    put_elem<DT>(e.tw, j, j < tail_n ? bits : ninf);
  }
}

// Clearing of the staging masks, which needs none of the row's loads: the
// kill mask spans kwords words (>= mw), its bytes from pad_byte on set
// (every id there removed); the seen mask spans swords words (>= mw).
__device__ __forceinline__ void stage_clear(const Lds &s, RowShared &sh, int kwords, int pad_byte,
                                            int swords) {
  const int tid = threadIdx.x;
  for (int w = tid; w < kwords; w += NT) {
    const int b0 = 4 * w;
    s.kmask[w] = b0 + 4 <= pad_byte ? 0u : b0 >= pad_byte ? ~0u : ~0u << (8 * (pad_byte - b0));
  }
  for (int w = tid; w < swords; w += NT) s.smask[w] = 0u;
  if (tid == 0) sh.n_coll = 0;
}

// Staging of a resident row in LDS once stage_clear has run (barriers that
// order LDS only):
//   kmask <- ids the registers drop: removed by a processor, or seen
//   smask <- alive seen ids; list_id <- those ids in id order
//   woff  <- list offset of every mask word
// Returns the list length, or -1 when the list does not fit: then the row's
// token is left pending for the streamed path and the caller returns.
__device__ __forceinline__ int stage(const SelectArgs &a, int row, const RowInfo &ri, const Lds &s,
                                     RowShared &sh, const int32_t *h, const Early &e,
                                     uint16_t *woff) {
  const int tid = threadIdx.x, V = a.V, mw = a.mw, L = ri.L;
  lds_barrier();
#pragma unroll
  for (int k = 0; k < kHpt; ++k) {
    const int v = e.hreg[k];
    if (tid + k * NT < L && v >= 0 && v < V) atomicOr(&s.smask[v >> 5], 1u << (v & 31));
  }
  for (int i = kHpt * NT + tid; i < L; i += NT) {  // long histories
    const int v = h[i];
    if (v >= 0 && v < V) atomicOr(&s.smask[v >> 5], 1u << (v & 31));
  }
  const int n = a.ngram;
  if (n > 0 && L >= n) {
    // Window i bans its last id when its first n-1 ids equal the last n-1
    // ids of the history (no_repeat_ngram_size).
    const int32_t *tl = h + (L - n + 1);
    for (int i = tid; i + n <= L; i += NT) {
      bool match = true;
      for (int j = 0; j < n - 1; ++j)
        if (h[i + j] != tl[j]) { match = false; break; }
      const int t = h[i + n - 1];
      if (match && t >= 0 && t < V) atomicOr(&s.kmask[t >> 5], 1u << (t & 31));
    }
  }
  const bool minlen_active = a.min_new > 0 ? (ri.new_tokens < a.min_new)
                                           : (a.min_length > 0 && L < a.min_length);
  if (minlen_active && tid < a.n_eos) {
    const int q = a.eos[tid];
    if (q >= 0 && q < V) atomicOr(&s.kmask[q >> 5], 1u << (q & 31));
  }
  lds_barrier();
  uint32_t aq[kMpt];
  int my_cnt = 0;
#pragma unroll
  for (int q = 0; q < kMpt; ++q) {
    const int w = tid * kMpt + q;
    aq[q] = 0u;
    if (w < mw) {
      const uint32_t K = s.kmask[w] | e.km[q] | (ri.begin_active ? e.kbeg[q] : 0u), S = s.smask[w];
      aq[q] = S & ~K;
      s.kmask[w] = K | S;
      s.smask[w] = aq[q];
      my_cnt += __popc(aq[q]);
    }
  }
  int n_list = 0;
  const int my_off = block_excl_scan_i32<NT, true>(my_cnt, sh.red_i32, &n_list);
  if (n_list > a.lcap) {  // too many seen ids for the list: the streamed path decides
    if (tid == 0) a.out_tokens[row] = kPending;
    return -1;
  }
  int o = my_off;
#pragma unroll
  for (int q = 0; q < kMpt; ++q) {
    if (tid * kMpt + q < mw) woff[tid * kMpt + q] = (uint16_t)o;
    uint32_t bits = aq[q];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      s.list_id[o++] = (tid * kMpt + q) * 32 + b;
    }
  }
  lds_barrier();
  return n_list;
}

}  // namespace res
}  // namespace tsel
