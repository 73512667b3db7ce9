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

// The same walk by one whole wave (every lane of the wave calls it; lane 0
// stores the result).  The individuals' masses are summed in runs of 64 by a
// wave scan and a ballot names the first position that reaches the goal; the
// tie group's share is solved in closed form as in the serial walk.  The
// partial sums are grouped differently from the serial walk's, so the two can
// differ by rounding where the goal falls within an ulp of a partial sum.
__device__ __forceinline__ void wave_walk(bool cut, double start, double goal, const BinView &bv,
                                 const uint64_t *okey, const float *oval, int pos_lim,
                                 WalkResult *out) {
  const int lane = threadIdx.x & (kWave - 1);
  const double e = (double)bv.e;
  const int na = bv.n_above, ni = bv.n_ind, ng = bv.n_group;
  double A = start;
  int kind = kFail, rank = -1, pos = -1, qk = -1;  // qk: the individual of a kInd result
  // Individuals [q0, q1) at positions po + q: true when the walk ends among them.
  auto run = [&](int q0, int q1, int po) -> bool {
    for (int b0 = q0; b0 < q1; b0 += kWave) {
      const int q = b0 + lane;
      const bool in = q < q1 && (cut || po + q <= pos_lim);
      const uint64_t inb = __ballot(in);
      if (inb == 0ull) return false;
      const double P = A + wave_incl_scan_f64_dpp(in ? (double)oval[q] : 0.0);
      const uint64_t hit = __ballot(in && (cut ? P >= goal : P > goal));
      const int f = hit ? __ffsll((unsigned long long)hit) - 1 : 63 - __clzll((long long)inb);
      kind = kInd;
      qk = b0 + f;
      pos = po + qk;
      const int src = hit ? f : kWave - 1;  // (uniform: read that lane directly)
      const unsigned long long pb = (unsigned long long)__double_as_longlong(P);
      const unsigned plo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)pb, src);
      const unsigned phi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(pb >> 32), src);
      A = __longlong_as_double((long long)(((unsigned long long)phi << 32) | plo));
      if (hit) return true;
    }
    return false;
  };
  if (cut) {
    // (a part that starts with the goal reached adds nothing)
    bool end = A >= goal || run(0, na, 0);
    if (!end && ng > 0) {
      if (A >= goal) {
        end = true;
      } else {
        // (a first guess by the reciprocal, by the division when the mass is
        // below the normal range; the loops below settle j exactly)
        const double q = bv.e >= 1.17549435e-38f ? (goal - A) * (double)__frcp_rn(bv.e) : (goal - A) / e;
        long long j = q < (double)ng ? (long long)ceil(q) : (long long)ng;
        if (j < 1) j = 1;
        while (j > 1 && A + (double)(j - 1) * e >= goal) --j;
        while (j < ng && A + (double)j * e < goal) ++j;
        kind = kGroup;
        if (j < ng) {
          rank = (int)j - 1;
          pos = na + (int)j - 1;
          A += (double)j * e;
          end = true;
        } else {
          A += (double)ng * e;
          rank = ng - 1;
          pos = na + ng - 1;
        }
      }
    }
    if (!end && !(A >= goal)) run(na, ni, ng);
  } else {
    bool end = run(0, na, 0);
    const int n_eff = pos_lim - na >= ng ? ng : pos_lim - na + 1;
    if (!end && n_eff > 0) {
      const double q = bv.e >= 1.17549435e-38f ? (goal - A) * (double)__frcp_rn(bv.e) : (goal - A) / e;
      long long j = q < (double)n_eff ? (long long)floor(q) : (long long)(n_eff - 1);
      if (j < 0) j = 0;
      while (j > 0 && A + (double)j * e > goal) --j;
      while (j < n_eff - 1 && A + (double)(j + 1) * e <= goal) ++j;
      kind = kGroup;
      rank = (int)j;
      pos = na + (int)j;
      if (A + (double)(j + 1) * e > goal) {
        end = true;
      } else {
        A += (double)n_eff * e;
        rank = n_eff - 1;
        pos = na + n_eff - 1;
      }
    }
    if (!end) run(na, ni, ng);
    A = 0.0;
  }
  if (lane == 0) {
    out->kind = kind;
    out->key = qk >= 0 ? okey[qk] : 0ull;
    out->rank = rank;
    out->pos = pos;
    out->acc = kind == kFail ? (cut ? A : 0.0) : A;
  }
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

// The small loads of a resident row, issued at the very start (none of them
// waits for the row's lengths): this thread's four history ids (slots 4 tid
// to 4 tid + 3; slots past the row's length are ignored later), its four
// kill-mask words and the row tail (V % EPC ids after the last whole chunk,
// as one more chunk).  All go through buffer resources, which read 0 past
// their end: no index is clamped, an absent mask or history is a resource
// of length 0, and no branch splits the loads, so that the row's chunks can
// later be waited for one at a time.
struct Early {
  int hreg[kHpt];
  uint32_t km[kMpt];    // bad words | suppress
  uint32_t kbeg[kMpt];  // begin-suppress, for rows where it applies
  uint32_t tw[4];       // the tail chunk as loaded, then (tail_words) as used
  uint32_t tlast;       // the last element of an odd bf16 row
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

template <int DT>
__device__ __forceinline__ void early_loads(const SelectArgs &a, int row, const char *rowp,
                                            Early &e) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  static_assert(kHpt == 4 && kMpt == 4, "four words per thread");
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, V = a.V;
  const int NG = V / EPC;
  const uint32_t mbytes = 4u * (uint32_t)a.mw;
  const int32_t *hp = a.hist_stride > 0 ? a.hist + (int64_t)row * a.hist_stride : a.lens;
  const u32x4_t hv = __builtin_amdgcn_raw_buffer_load_b128(
      buf_rsrc(hp, 4u * (uint32_t)max(a.hist_stride, 0)), tid * 16, 0, 0);
  const u32x4_t m0 = __builtin_amdgcn_raw_buffer_load_b128(
      buf_rsrc(a.bad_mask ? (const void *)a.bad_mask : a.lens, a.bad_mask ? mbytes : 0u), tid * 16, 0, 0);
  const u32x4_t m1 = __builtin_amdgcn_raw_buffer_load_b128(
      buf_rsrc(a.sup_mask ? (const void *)a.sup_mask : a.lens, a.sup_mask ? mbytes : 0u), tid * 16, 0, 0);
  const u32x4_t m2 = __builtin_amdgcn_raw_buffer_load_b128(
      buf_rsrc(a.begin_mask ? (const void *)a.begin_mask : a.lens, a.begin_mask ? mbytes : 0u), tid * 16, 0, 0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    e.hreg[k] = (int)hv[k];
    e.km[k] = m0[k] | m1[k];
    e.kbeg[k] = m2[k];
  }
  // the tail: every lane reads the same partial chunk, its whole words by
  // one 16-byte load through a resource that ends at the row's last whole
  // word (the words past it read as 0), and the last element of an odd bf16
  // row by itself; elements past the row become -inf
  const int tail_n = V - NG * EPC;
  const uint32_t row_bytes = (uint32_t)V * (DT == 1 ? 2u : 4u);
  const u32x4_t tv = __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(rowp, row_bytes & ~3u), NG * 16, 0, 0);
  e.tlast = DT == 1 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(buf_rsrc(rowp, row_bytes), (V - 1) * 2, 0, 0) : 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) e.tw[q] = tv[q];
  (void)tail_n;
}

// The tail chunk made whole, where it is used: the empty asm keeps the
// compiler from reading the loaded words (and so waiting for every load
// before them) right after they were asked for, ahead of the row's loads.
template <int DT>
__device__ __forceinline__ void tail_words(Early &e, int V) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  asm volatile("" : "+v"(e.tw[0]), "+v"(e.tw[1]), "+v"(e.tw[2]), "+v"(e.tw[3]), "+v"(e.tlast));
  const int tail_n = V - (V / EPC) * EPC;
  const uint32_t ninf = DT == 1 ? 0xFF80u : 0xFF800000u;
#pragma unroll
  for (int j = 0; j < EPC; ++j) {
    if (j >= tail_n) put_elem<DT>(e.tw, j, ninf);
    else if (DT == 1 && (V & 1) && j == tail_n - 1) put_elem<DT>(e.tw, j, e.tlast);
  }
}

// Clearing of the staging masks, which needs none of the row's loads: the
// kill mask spans kwords words (>= mw), its bytes from pad_byte on set
// (every id there removed); the seen mask spans swords words (>= mw).
__device__ __forceinline__ void stage_clear(const Lds &s, RowShared &sh, int kwords, int pad_byte,
                                            int swords) {
  const int tid = threadIdx.x;
  // (16 bytes a store; both masks start 16-byte aligned and span whole
  // multiples of 4 words, rounded up here)
  for (int w4 = tid; w4 < (kwords + 3) / 4; w4 += NT) {
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b0 = 16 * w4 + 4 * q;
      v[q] = b0 + 4 <= pad_byte ? 0u : b0 >= pad_byte ? ~0u : ~0u << (8 * (pad_byte - b0));
    }
    reinterpret_cast<uint4 *>(s.kmask)[w4] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  for (int w4 = tid; w4 < (swords + 3) / 4; w4 += NT)
    reinterpret_cast<uint4 *>(s.smask)[w4] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) sh.n_coll = 0;
}

// Staging of a resident row in LDS once stage_clear has run, in three steps
// that a kernel may run between the counts of its row's first chunks (each
// ends in a barrier that orders LDS only):
//   stage_marks: seen bits, n-gram bans, the eos ban of the minimum lengths;
//   stage_merge: kmask <- ids the registers drop (removed by a processor, or
//                seen); smask <- alive seen ids; the list's size and this
//                thread's offset in it;
//   stage_list:  list_id <- the alive seen ids in id order; woff <- the list
//                offset of every mask word.
struct StageState {
  uint32_t aq[kMpt];  // this thread's alive seen words
  int my_off;         // its first list slot
  int n_list;         // the list's length
};

__device__ __forceinline__ void stage_marks(const SelectArgs &a, const RowInfo &ri, const Lds &s,
                                            const int32_t *h, const Early &e) {
  const int tid = threadIdx.x, V = a.V, L = ri.L;
  lds_barrier();
#pragma unroll
  for (int k = 0; k < kHpt; ++k) {
    const int v = e.hreg[k];
    if (tid * kHpt + k < L && v >= 0 && v < V) atomicOr(&s.smask[v >> 5], 1u << (v & 31));
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
}

__device__ __forceinline__ void stage_merge(const SelectArgs &a, const RowInfo &ri, const Lds &s,
                                            RowShared &sh, const Early &e, StageState &st) {
  const int tid = threadIdx.x, mw = a.mw;
  // (a thread's four words in one 16-byte read and write per mask; words
  // past mw, inside the masks' rounded-up span, hold no seen id, and their
  // early-loaded words read as 0, so taking them along changes nothing)
  int my_cnt = 0;
#pragma unroll
  for (int q = 0; q < kMpt; ++q) st.aq[q] = 0u;
  if (tid * kMpt < mw) {
    const uint4 k4 = reinterpret_cast<const uint4 *>(s.kmask)[tid];
    const uint4 s4 = reinterpret_cast<const uint4 *>(s.smask)[tid];
    const uint32_t kq[kMpt] = {k4.x, k4.y, k4.z, k4.w}, sq[kMpt] = {s4.x, s4.y, s4.z, s4.w};
    uint32_t kn[kMpt];
#pragma unroll
    for (int q = 0; q < kMpt; ++q) {
      const uint32_t K = kq[q] | e.km[q] | (ri.begin_active ? e.kbeg[q] : 0u);
      st.aq[q] = sq[q] & ~K;
      kn[q] = K | sq[q];
      my_cnt += __popc(st.aq[q]);
    }
    reinterpret_cast<uint4 *>(s.kmask)[tid] = make_uint4(kn[0], kn[1], kn[2], kn[3]);
    reinterpret_cast<uint4 *>(s.smask)[tid] = make_uint4(st.aq[0], st.aq[1], st.aq[2], st.aq[3]);
  }
  // Exclusive prefix of the counts over the workgroup: one barrier (the
  // wave totals' slots were last read before the barrier above), the
  // totals' prefix by row moves, read out of its lanes.
  constexpr int NW_ = NT / kWave;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const int incl = wave_incl_scan_i32(my_cnt);
  if (lane == kWave - 1) sh.red_i32[wid] = incl;
  lds_barrier();
  const int wsum = lane < NW_ ? sh.red_i32[lane] : 0;
  const int wincl = wave_incl_scan_i32(wsum);
  st.my_off = __builtin_amdgcn_readlane(wincl - wsum, uni(wid)) + incl - my_cnt;
  st.n_list = __builtin_amdgcn_readlane(wincl, NW_ - 1);
}

// Returns the list length, or -1 when the list does not fit: then the row's
// token is left pending for the streamed path and the caller returns.
__device__ __forceinline__ int stage_list(const SelectArgs &a, int row, const Lds &s,
                                          uint16_t *woff, const StageState &st) {
  const int tid = threadIdx.x, mw = a.mw;
  if (st.n_list > a.lcap) {  // too many seen ids for the list: the streamed path decides
    if (tid == 0) a.out_tokens[row] = kPending;
    return -1;
  }
  int o = st.my_off;
#pragma unroll
  for (int q = 0; q < kMpt; ++q) {
    if (tid * kMpt + q < mw) woff[tid * kMpt + q] = (uint16_t)o;
    uint32_t bits = st.aq[q];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      s.list_id[o++] = (tid * kMpt + q) * 32 + b;
    }
  }
  lds_barrier();
  return st.n_list;
}

// The three steps in a row.
__device__ __forceinline__ int stage(const SelectArgs &a, int row, const RowInfo &ri, const Lds &s,
                                     RowShared &sh, const int32_t *h, const Early &e,
                                     uint16_t *woff) {
  stage_marks(a, ri, s, h, e);
  StageState st;
  stage_merge(a, ri, s, sh, e, st);
  return stage_list(a, row, s, woff, st);
}

}  // namespace res
}  // namespace tsel
