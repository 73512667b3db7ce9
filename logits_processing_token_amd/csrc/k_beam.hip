// k_beam.hip -- one step of beam search over the logits of num_beams rows
// per prompt ("Transmuter.Generation (transmuter v2.0.0)", the beam
// paragraph under "Log-probabilities"): each beam row takes the log-softmax
// of its logits, the processors act on that with removed ids at the
// smallest finite value, and the beam's score is added, a score never going
// below the smallest finite value; of a prompt's num_beams * V candidates
// the best K = max(2, 1 + eos ids) * num_beams are kept.  On the first step
// only beam 0 of a prompt counts; a padding beam row (length 0) gives none.
//
// A candidate (beam j, id v) of a prompt has the flattened index
// e = j * V + v and the 64-bit key (ordered score << 32) | (2^32 - 1 - e):
// keys are unique and order candidates as the step does (score descending,
// then e ascending), so the best K are the K largest keys.  No key is 0, which
// marks "no candidate".
//
//  * k_beam_rows, one workgroup per beam row: the seen and removed ids as two
//    bitmasks in LDS; a logit bound from a sample, every lane's first chunk
//    (K of its ids neither removed nor seen lie at or above it); one pass
//    for the row's largest logit m and log(sum exp(x - m)) in binary64
//    (exp_nonpos for the terms) that also keeps on chip the ids at or above
//    the bound; then the row's best K keys among those, rescored.  A bf16
//    row's pass counts each logit into a bin per bf16 value and takes one
//    exponential per bin.  When the bound fails (too many kept, a sample
//    smaller than K, or rounding that could tie a left-out id with the
//    sample's K-th), the best K come from a second pass over the row,
//    bounded by the sample's K-th key.  Nothing of size V is written.
//  * k_beam_merge, one workgroup per prompt: the best K of its num_beams * K
//    row keys, written as score, beam and id (k_beam_merge_wave, one wave,
//    when those keys number at most 64).
//
// The selections: a short kept list (at most a quarter of the workgroup's
// lanes) is ranked on chip, each key's rank the count of larger keys; for
// K up to the number of waves, a longer one by rounds of wave maxima; any
// other set by a radix select over the keys, 12 bits then 13 at a time from
// the top, stopping as soon as the keys at or above the current prefix
// number at most kSelCap, which are then ranked on chip.

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "tsel_device.hpp"
#include "k_vkey.hpp"
#include "tsel_internal.hpp"

namespace tsel {
namespace {

constexpr int kBT = kBeamThreads;

struct SelShared {
  int wsum[kBT / kWave];
  int total, digit, above, cnt, nc;
};

__device__ __forceinline__ uint32_t ordered32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ bool has_bit(const uint32_t *m, int v) {
  return (m[v >> 5] >> (v & 31)) & 1u;
}

// The wave's largest key, on every lane: row moves (quad swaps, half-row and
// row mirrors, then the row broadcasts) on both halves, read from the last
// lane.
template <int C, int RM>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, C, RM, 0xF, false);
  const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, C, RM, 0xF, false);
  const uint64_t w = ((uint64_t)h2 << 32) | l2;
  return w > v ? w : v;
}
__device__ __forceinline__ uint64_t wave_max_u64_uni(uint64_t v) {
  v = dpp_max_u64<0xB1, 0xF>(v);
  v = dpp_max_u64<0x4E, 0xF>(v);
  v = dpp_max_u64<0x141, 0xF>(v);
  v = dpp_max_u64<0x140, 0xF>(v);
  v = dpp_max_u64<0x142, 0xA>(v);
  v = dpp_max_u64<0x143, 0xC>(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, kWave - 1);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), kWave - 1);
  return ((uint64_t)hi << 32) | lo;
}

// The largest min(K, present keys) of the keys visit(f) passes to f, one
// call per key and thread (0 = absent), each passed to emit(rank, key), rank
// 0 the largest; returns how many.  Every thread of the workgroup calls.
// hist: kBeamSelBins words; cand: kSelCap keys.
// direct: first gather every key on chip in one pass, ranked there when
// they number at most kSelCap (else the radix passes follow).
template <class Visit, class EmitFn>
__device__ __forceinline__ int select_top(int K, Visit visit, EmitFn emit, uint32_t *hist,
                                          uint64_t *cand, SelShared &ss, bool direct = false) {
  const int tid = threadIdx.x;
  if (direct) {
    if (tid == 0) ss.nc = 0;
    __syncthreads();
    visit([&](uint64_t k) {
      if (k != 0ull) {
        const int slot = atomicAdd(&ss.nc, 1);
        if (slot < kSelCap) cand[slot] = k;
      }
    });
    __syncthreads();
    const int nc = ss.nc;
    __syncthreads();  // (ss is written again below)
    if (nc <= kSelCap) {
      const int keff = nc < K ? nc : K;
      for (int j = tid; j < nc; j += kBT) {
        const uint64_t kj = cand[j];
        int r = 0;
        for (int q = 0; q < nc; ++q) r += cand[q] > kj;
        if (r < keff) emit(r, kj);
      }
      return keff;
    }
  }
  uint64_t prefix = 0ull, pmask = 0ull;
  int need = 0, above = 0, keff = 0;
  for (int pass = 0; pass < 5; ++pass) {
    const int width = pass == 0 ? 12 : 13;
    const int shift = 52 - 13 * pass;
    const int nbins = 1 << width;
    for (int d = tid; d < nbins; d += kBT) hist[d] = 0u;
    __syncthreads();
    visit([&](uint64_t k) {
      if (k != 0ull && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & (nbins - 1)], 1u);
    });
    __syncthreads();
    // thread t holds bins top, top-1, ..., the t-th group from the top
    const int per = nbins / kBT;
    const int top = nbins - 1 - tid * per;
    int s = 0;
    for (int i = 0; i < per; ++i) s += (int)hist[top - i];
    int total = 0;
    const int excl = block_excl_scan_i32<kBT>(s, ss.wsum, &total);
    if (pass == 0) {
      keff = total < K ? total : K;
      if (keff == 0) return 0;
      need = keff;
    }
    if (excl < need && need <= excl + s) {  // (exactly one thread)
      int acc = excl;
      for (int i = 0; i < per; ++i) {
        const int c = (int)hist[top - i];
        if (acc + c >= need) {
          ss.digit = top - i;
          ss.above = acc;
          ss.cnt = c;
          break;
        }
        acc += c;
      }
    }
    if (tid == 0) ss.nc = 0;
    __syncthreads();
    above += ss.above;
    need -= ss.above;
    prefix |= (uint64_t)ss.digit << shift;
    pmask |= (uint64_t)(nbins - 1) << shift;
    const int cnt = ss.cnt;
    __syncthreads();  // (ss is written again on the next pass)
    if (above + cnt <= kSelCap) break;  // (after the last pass: above + cnt = keff)
  }
  // the keys at or above the prefix: `above` with a larger prefix, then the
  // ones sharing it, the keff-th largest among them
  visit([&](uint64_t k) {
    if (k != 0ull && (k & pmask) >= prefix) {
      const int slot = atomicAdd(&ss.nc, 1);
      if (slot < kSelCap) cand[slot] = k;
    }
  });
  __syncthreads();
  const int nc = ss.nc < kSelCap ? ss.nc : kSelCap;
  for (int j = tid; j < nc; j += kBT) {
    const uint64_t kj = cand[j];
    int r = 0;
    for (int q = 0; q < nc; ++q) r += cand[q] > kj;
    if (r < keff) emit(r, kj);
  }
  return keff;
}

// The row's whole 16-byte chunks, each passed to consume(c, g) (g the
// chunk's index) by the lane that loads it: lane t takes chunks t, t + kBT,
// ...  in batches of kVB per lane, the batches' registers alternating
// between two sets so that a batch's loads fly while the one before it is
// consumed.  Buffer loads read 0 past the chunks, so no branch guards them
// and the wait before a batch is for that batch alone.  p holds batch 0,
// asked for by the caller (load_batch(rs, p, 0)).
constexpr int kVB = 4;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const char *rowp, int NG) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(rowp), (short)0, NG * 16, 0x00020000);
}
__device__ __forceinline__ void load_batch(__amdgpu_buffer_rsrc_t rs, u32x4_t (&d)[kVB], int b) {
#pragma unroll
  for (int u = 0; u < kVB; ++u)
    d[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((b * kVB + u) * kBT + (int)threadIdx.x) * 16, 0, 0);
}
template <class C>
__device__ __forceinline__ void stream_chunks(__amdgpu_buffer_rsrc_t rs, int NG, u32x4_t (&p)[kVB],
                                              C &&consume) {
  constexpr int S = kBT * kVB;
  const int tid = threadIdx.x;
  const int nb = (NG + S - 1) / S;
  u32x4_t q[kVB];
  auto use = [&](const u32x4_t (&d)[kVB], int b) {
#pragma unroll
    for (int u = 0; u < kVB; ++u) {
      const int g = b * S + u * kBT + tid;
      if (g < NG) consume(d[u], g);
    }
  };
  for (int b = 0; b < nb; b += 2) {
    load_batch(rs, q, b + 1);
    use(p, b);
    load_batch(rs, p, b + 2);
    use(q, b + 1);
  }
}

// f(v, x) for every element v of a row (16-byte rows: whole chunks of 8
// bf16 or 4 fp32, then the tail), x widened to binary32; p: the row's batch
// 0, asked for through rs = chunk_rsrc(rowp, V / (8 or 4)).
template <class F>
__device__ __forceinline__ void visit_row(const char *rowp, bool bf16, int V, __amdgpu_buffer_rsrc_t rs,
                                          u32x4_t (&p)[kVB], F &&f) {
  const int tid = threadIdx.x;
  const int epc = bf16 ? 8 : 4;
  const int NG = V / epc;
  stream_chunks(rs, NG, p, [&](const u32x4_t &c, int g) {
    if (bf16) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        f(g * 8 + j, (j & 1) ? __uint_as_float(c[j >> 1] & 0xFFFF0000u)
                             : __uint_as_float(c[j >> 1] << 16));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) f(g * 4 + j, __uint_as_float(c[j]));
    }
  });
  for (int v = NG * epc + tid; v < V; v += kBT)
    f(v, bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(rowp)[v] << 16)
              : reinterpret_cast<const float *>(rowp)[v]);
}
template <class F>
__device__ __forceinline__ void visit_row(const char *rowp, bool bf16, int V, F &&f) {
  const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(rowp, V / (bf16 ? 8 : 4));
  u32x4_t p[kVB];
  load_batch(rs, p, 0);
  visit_row(rowp, bf16, V, rs, p, f);
}

// The counting pass of a bf16 row: every element adds 1 to the bin of its
// value key k (vkey), clamped to [lo, hi]: bins[k - lo] (bin 0 takes the
// keys below lo, bin hi - lo the keys at or above hi).  A 16-byte chunk
// with an element on a near-zero key or at or above `spec` has
// special(v, x, k, t) called for each of those elements by the lane that
// holds it (t = 0 on the near-zero keys), and so has every element of the
// row tail.  rs, p: as visit_row's.
template <class Special>
__device__ __forceinline__ void count_row_bf16(const char *rowp, int V, __amdgpu_buffer_rsrc_t rs,
                                               u32x4_t (&p)[kVB], uint32_t *bins, uint32_t lo,
                                               uint32_t hi, uint32_t spec, Special &&special) {
  const int tid = threadIdx.x;
  const int NG = V / 8;
  auto key = [&](uint32_t hw, uint32_t &t) {  // hw: the bf16 pattern in the low 16 bits
    const uint32_t m = hw & 0x7FFFu;
    t = m > kZoneMag ? m - kZoneMag : 0u;
    const uint32_t sgn = 0u - ((hw >> 15) & 1u);  // all ones for a negative value
    return (t ^ sgn) + 0x8000u;                    // 0x8000 + t, or 0x7FFF - t
  };
  stream_chunks(rs, NG, p, [&](const u32x4_t &w, int g) {
    bool odd = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t t;
      const uint32_t k = key((j & 1) ? (w[j >> 1] >> 16) : w[j >> 1], t);
      atomicAdd(&bins[min(max(k, lo), hi) - lo], 1u);
      odd |= (k >= spec) | (t == 0u);
    }
    if (odd)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t hw = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
        uint32_t t;
        const uint32_t k = key(hw, t);
        if (k >= spec || t == 0u) special(g * 8 + j, __uint_as_float(hw << 16), k, t);
      }
  });
  for (int v = NG * 8 + tid; v < V; v += kBT) {  // (the row tail: every element special)
    const uint32_t hw = reinterpret_cast<const uint16_t *>(rowp)[v];
    uint32_t t;
    const uint32_t k = key(hw, t);
    atomicAdd(&bins[min(max(k, lo), hi) - lo], 1u);
    special(v, __uint_as_float(hw << 16), k, t);
  }
}

}  // namespace

__global__ __launch_bounds__(kBT, 1) void k_beam_rows(BeamArgs a) {
  extern __shared__ __align__(16) uint32_t bsm[];
  __shared__ float rmax[kBT / kWave];
  __shared__ double rsum[kBT / kWave];
  __shared__ SelShared ss;
  const SelectArgs &s = a.s;
  const int r = blockIdx.x, tid = threadIdx.x, V = s.V, K = a.width;
  const int beam = r % a.nb;
  uint64_t *keys_out = a.row_keys + (int64_t)r * K;
  const char *rowp = s.logits + (int64_t)r * s.row_bytes;
  const bool bf16 = s.dtype == 1;
  const int mw = (V + 31) / 32;
  const int epc = bf16 ? 8 : 4;
  const int NGs = V / epc;
  const int32_t *h = s.hist + (int64_t)r * s.hist_stride;
  // Asked for before the row's lengths arrive: the first history ids and
  // the static masks' first words, four per lane, then the row's first
  // batch of chunks (its first chunk per lane is the sample below; the sum
  // pass starts on the batch), which stays in flight while the masks are
  // built (the barriers up to the sample order LDS alone).
  // (through buffer resources, which read 0 past their end, so that no
  // branch splits the loads: an absent mask is a resource of length 0)
  auto rsrc = [&](const void *q, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(q ? q : (const void *)s.lens), (short)0,
                                             q ? bytes : 0, 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t hrs = rsrc(s.hist_stride > 0 ? h : nullptr, 4 * s.hist_stride);
  const __amdgpu_buffer_rsrc_t brs = rsrc(s.bad_mask, 4 * mw), srs = rsrc(s.sup_mask, 4 * mw);
  int hv0[4];
  uint32_t km0[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = tid + u * kBT;
    hv0[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(hrs, 4 * i, 0, 0);
    km0[u] = __builtin_amdgcn_raw_buffer_load_b32(brs, 4 * i, 0, 0) |
             __builtin_amdgcn_raw_buffer_load_b32(srs, 4 * i, 0, 0);
  }
  auto static_word = [&](int w) {
    return __builtin_amdgcn_raw_buffer_load_b32(brs, 4 * w, 0, 0) |
           __builtin_amdgcn_raw_buffer_load_b32(srs, 4 * w, 0, 0);
  };
  const __amdgpu_buffer_rsrc_t rrs = chunk_rsrc(rowp, NGs);
  u32x4_t b0[kVB];
  load_batch(rrs, b0, 0);
  const int L = s.lens[r], P = s.lens[s.B + r], M = s.lens[2 * s.B + r];
  const float s_beam = a.beam_scores[r];
  if ((a.first_step && beam > 0) || L <= 0) {  // no candidates
    for (int i = tid; i < K; i += kBT) keys_out[i] = 0ull;
    return;
  }
  uint32_t *seen = bsm, *kill = bsm + mw;
  uint32_t *hist = bsm + ((2 * mw + 3) & ~3);
  uint64_t *cand = reinterpret_cast<uint64_t *>(hist + kBeamSelBins);
  int32_t *kid = reinterpret_cast<int32_t *>(cand + kSelCap);  // ids the sum pass keeps
  float *kx = reinterpret_cast<float *>(kid + kSelCap);        // and their logits
  __shared__ int keep_n;
  __shared__ float xf_s;
  __shared__ float wmax_s[2][kBT / kWave];
  constexpr int NW = kBT / kWave;
  const int lane = tid & (kWave - 1);
  const int new_tokens = L - P;
  const bool begin_active =
      s.begin_mask != nullptr && new_tokens == ((s.forced_bos >= 0 && P == 1) ? 1 : 0);
  int forced = -1;
  if (s.forced_bos >= 0 && L == 1) forced = s.forced_bos;
  if (s.forced_eos >= 0 && L == M - 1) forced = s.forced_eos;
  const int Lh = L < s.hist_stride ? L : s.hist_stride;  // (ids past the stride are not the row's)
  // ---- the processors' masks (LDS): seen ids; the static masks, n-gram and
  // minimum-length bans as removals (the removals start as the static
  // masks) ----
  for (int w0 = tid; w0 < mw; w0 += 4 * kBT) {
    uint32_t k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int w = w0 + u * kBT;
      k[u] = 0u;
      if (w < mw) {
        k[u] = w0 == tid ? km0[u] : static_word(w);
        if (begin_active) k[u] |= s.begin_mask[w];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int w = w0 + u * kBT;
      if (w < mw) {
        seen[w] = 0u;
        kill[w] = k[u];
      }
    }
  }
  if (tid == 0) {
    keep_n = 0;
    xf_s = -INFINITY;
  }
  lds_barrier();
  if (forced < 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (tid + u * kBT < Lh && hv0[u] >= 0 && hv0[u] < V)
        atomicOr(&seen[hv0[u] >> 5], 1u << (hv0[u] & 31));
    for (int i0 = tid + 4 * kBT; i0 < Lh; i0 += 4 * kBT) {
      int hv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) hv[u] = i0 + u * kBT < Lh ? h[i0 + u * kBT] : -1;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (hv[u] >= 0 && hv[u] < V) atomicOr(&seen[hv[u] >> 5], 1u << (hv[u] & 31));
    }
    const int n = s.ngram;
    if (n > 0 && Lh >= n) {  // window i bans its last id when its head is the history's tail
      const int32_t *tl = h + (Lh - n + 1);
      for (int i = tid; i + n <= Lh; i += kBT) {
        bool match = true;
        for (int j = 0; j < n - 1; ++j)
          if (h[i + j] != tl[j]) { match = false; break; }
        const int t = h[i + n - 1];
        if (match && t >= 0 && t < V) atomicOr(&kill[t >> 5], 1u << (t & 31));
      }
    }
    const bool minlen_active =
        s.min_new > 0 ? (new_tokens < s.min_new) : (s.min_length > 0 && L < s.min_length);
    if (minlen_active && tid < s.n_eos) {
      const int e = s.eos[tid];
      if (e >= 0 && e < V) atomicOr(&kill[e >> 5], 1u << (e & 31));
    }
  }
  lds_barrier();
  bool forced_alive = forced >= 0 && forced < V;
  if (forced_alive && s.sup_mask && has_bit(s.sup_mask, forced)) forced_alive = false;
  if (forced_alive && begin_active && has_bit(s.begin_mask, forced)) forced_alive = false;
  const u32x4_t c0 = b0[0];
  auto elem = [&](const u32x4_t &c, int j) {
    return bf16 ? ((j & 1) ? __uint_as_float(c[j >> 1] & 0xFFFF0000u) : __uint_as_float(c[j >> 1] << 16))
                : __uint_as_float(c[j]);
  };
  // ---- from the sample: M0, the largest logit of the first chunks and
  // the row tail (the log-softmax's provisional shift), and the largest
  // logit among the sample ids that are neither removed nor seen of each of
  // NW groups of lanes ----
  float m0 = -INFINITY, me = -INFINITY;
  if (tid < NGs) {
    // (a lane's epc ids lie in one word of each mask)
    const int w = (tid * epc) >> 5, b0 = (tid * epc) & 31;
    const uint32_t out = (kill[w] | seen[w]) >> b0;
    for (int j = 0; j < epc; ++j) {
      const float x = elem(c0, j);
      m0 = fmaxf(m0, x);
      if (x > -INFINITY && !((out >> j) & 1u)) me = fmaxf(me, x);
    }
  }
  for (int v = NGs * epc + tid; v < V; v += kBT)  // (the row tail)
    m0 = fmaxf(m0, bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(rowp)[v] << 16)
                        : reinterpret_cast<const float *>(rowp)[v]);
  float *lme = reinterpret_cast<float *>(cand);  // (free until the selection)
  lme[tid] = me;
  {
    const float wm = wave_max_f32_uni(m0);
    if (lane == 0) wmax_s[0][tid / kWave] = wm;
  }
  lds_barrier();
  {
    // group w: the lanes t with t mod NW = w, whose chunks spread over the
    // sample (so that ids in order of their logits do not crowd one group)
    const float ge = wave_max_f32_uni(lme[tid / kWave + NW * lane]);
    if (lane == 0) wmax_s[1][tid / kWave] = ge;
  }
  lds_barrier();
  float M0 = -INFINITY;
#pragma unroll
  for (int q = 0; q < NW; ++q) M0 = fmaxf(M0, wmax_s[0][q]);
  // ---- a logit bound from the sample, xf: K ids of the sample that are
  // neither removed nor seen have logits at or above it.  Those K score
  // their plain log-probability, so an id whose logit lies below xf far
  // enough that even its plain score is lower (checked once the log-softmax
  // is known) cannot be among the row's best K: the sum pass keeps the ids
  // at or above xf less a small slack, on chip.  For K up to the number of
  // groups, xf is the K-th largest of the groups' maxima (each held by an id
  // of its own group); else the K-th largest of the sample itself. ----
  bool bounded = false;
  float xthr = INFINITY, xf = -INFINITY;
  if (forced < 0) {
    if (K <= NW) {
      const float wv = lane < NW ? wmax_s[1][lane] : -INFINITY;
      int rank = 0;  // (equal maxima ranked by group)
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const float o = wmax_s[1][q];
        rank += (o > wv || (o == wv && q < lane)) ? 1 : 0;
      }
      const uint64_t hit = __ballot(lane < NW && rank == K - 1);  // (one lane)
      xf = wmax_s[1][__ffsll((unsigned long long)hit) - 1];
    } else {
      const int ns = select_top(
          K,
          [&](auto &&f) {
            if (tid < NGs)
              for (int j = 0; j < epc; ++j) {
                const int v = tid * epc + j;
                const float x = elem(c0, j);
                if (x > -INFINITY && !has_bit(kill, v) && !has_bit(seen, v))
                  f(((uint64_t)ordered32(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v));
              }
          },
          [&](int rank, uint64_t k) {
            if (rank == K - 1) xf_s = unordered32((uint32_t)(k >> 32));
          },
          hist, cand, ss);
      __syncthreads();
      xf = ns == K ? xf_s : -INFINITY;
    }
    bounded = xf > -INFINITY;
    if (bounded) xthr = xf - fmaxf(fabsf(xf) * 0x1p-12f, 0x1p-20f);
  }
  float mloc = -INFINITY;
  double sum = 0.0;
  const double dM0 = M0 > -INFINITY ? (double)M0 : 0.0;
  // e^d: exp_nonpos for d <= 0; above (a logit over M0), e^(d - 700) e^700,
  // enough up to d = 700 (past that the sum is taken again against the
  // row's maximum): one polynomial either way.
  auto term = [&](double d) {
    const bool neg = d <= 0.0;
    const double e = exp_nonpos(neg ? d : fmin(d, 700.0) - 700.0);
    return neg ? e : e * 0x1.d945df4f8ec8ep+1009;  // (e^700)
  };
  // bf16 rows: each logit adds 1 to a bin per bf16 value, and the sum takes
  // one exponential per bin (count times it) instead of one per logit.  The
  // bins run from the value 746 below M0 (every term below underflows to 0)
  // up; near-zero logits (one key for a range of values) and logits past
  // the bins take their own term.  The select's radix bins are free during
  // the pass and hold two copies (by lane parity).
  static_assert(2 * kVStride <= kBeamSelBins, "two copies of the value bins");
  const bool vsum = bf16 && M0 > -INFINITY;
  uint32_t klo = 0u, khi = 0u;
  uint32_t *vbl = hist + (tid & 1) * kVStride;
  if (vsum) {
    klo = max(vkey_floor(M0 - 746.0f), kKeyLowFinite);
    khi = klo + (uint32_t)(kVBins - 1);
    for (int i = tid; i < 2 * kVStride; i += kBT) hist[i] = 0u;
    __syncthreads();
  }
  auto keep = [&](int v, float x) {
    if (x >= xthr) {
      const int slot = atomicAdd(&keep_n, 1);
      if (slot < kSelCap) {
        kid[slot] = v;
        kx[slot] = x;
      }
    }
  };
  if (vsum) {
    // the keys at or above kspec include every logit at or above xthr
    const uint32_t kspec = min(vkey_floor(xthr), khi);
    count_row_bf16(rowp, V, rrs, b0, vbl, klo - 1u, khi, kspec, [&](int v, float x, uint32_t k, uint32_t t) {
      if (t == 0u || k >= khi) {  // (not in a bin the sum reads)
        mloc = fmaxf(mloc, x);
        sum += term((double)x - dM0);
      }
      keep(v, x);
    });
    __syncthreads();
    for (int b = 1 + tid; b < kVBins; b += kBT) {
      const uint32_t n = hist[b] + hist[kVStride + b];
      const uint32_t kb = klo + (uint32_t)b - 1u;
      if (n != 0u && kb != kKeyZoneNeg && kb != kKeyZonePos) {
        const float xb = vkey_value(kb);
        mloc = fmaxf(mloc, xb);
        sum += (double)n * term((double)xb - dM0);
      }
    }
  } else {
    visit_row(rowp, bf16, V, rrs, b0, [&](int v, float x) {  // (-inf adds 0)
      mloc = fmaxf(mloc, x);
      sum += term((double)x - dM0);
      keep(v, x);
    });
  }
  const float Mx = block_max_f32<kBT>(mloc, rmax);
  double S;
  if (Mx > -INFINITY && (double)Mx - dM0 > 700.0) {  // (rare: far above the first chunks)
    sum = 0.0;
    visit_row(rowp, bf16, V, [&](int, float x) { sum += exp_nonpos((double)x - (double)Mx); });
    S = block_sum_f64<kBT>(sum, rsum);
  } else {
    S = block_sum_f64<kBT>(sum, rsum) * (Mx > -INFINITY ? exp(dM0 - (double)Mx) : 1.0);
  }
  const bool any = Mx > -INFINITY;
  const float lsf = any ? (float)log(S) : 0.0f;
  const uint32_t flat0 = (uint32_t)beam * (uint32_t)V;
  // A candidate's ordered score bits: plain_bits for an id neither removed
  // nor seen, true_bits for any id (the forced row, the removal, the
  // penalty); then its key.
  auto finish = [&](float y) -> uint32_t {
    float c = y + s_beam;
    if (!(c >= -FLT_MAX)) c = -FLT_MAX;  // never below the smallest finite value
    if (c == 0.0f) c = 0.0f;             // (-0 and +0 are one score)
    return ordered32(c);
  };
  auto base = [&](float x) { return (any && x > -INFINITY) ? (x - Mx) - lsf : x; };
  auto plain_bits = [&](float x) -> uint32_t { return finish(base(x)); };
  auto true_bits = [&](int v, float x) -> uint32_t {
    float y;
    if (forced >= 0) {
      y = (forced_alive && v == forced) ? 0.0f : -FLT_MAX;
    } else {
      y = base(x);
      if (has_bit(kill, v)) {
        y = -FLT_MAX;
      } else if (s.rep != 1.0f && has_bit(seen, v)) {
        y = penalize(y, s.rep);
      }
    }
    return finish(y);
  };
  auto key_of = [&](int v, uint32_t ob) -> uint64_t {
    return ((uint64_t)ob << 32) | (uint64_t)(0xFFFFFFFFu - (flat0 + (uint32_t)v));
  };
  auto emit_row = [&](int rank, uint64_t k) { keys_out[rank] = k; };
  int keff;
  if (forced >= 0) {
    // every id but the forced one scores alike: the best K are among the
    // forced id and the K lowest others
    keff = select_top(
        K,
        [&](auto &&f) {
          for (int v = tid; v <= K && v < V; v += kBT)
            if (v != forced) f(key_of(v, true_bits(v, 0.0f)));
          if (tid == 0 && forced < V) f(key_of(forced, true_bits(forced, 0.0f)));
        },
        emit_row, hist, cand, ss);
  } else if (bounded && keep_n <= kSelCap && plain_bits(nextafterf(xthr, -INFINITY)) < plain_bits(xf)) {
    // Every id left out of the sum pass's list scores below the sample's K
    // ids (whose scores are plain): the best K are among the list, rescored,
    // and (a penalty below 1 raising them) the seen ids below the bound.
    const int nk = keep_n;
    const bool raise = s.rep < 1.0f;
    if (!raise && nk <= kBT / 4) {
      // The list alone, a key a lane: a key's rank is the count of larger
      // keys, counted by kBT / nk lanes, a share of the list each.
      if (tid < nk) cand[tid] = key_of(kid[tid], true_bits(kid[tid], kx[tid]));
      uint32_t *rk = hist;  // (the bins, read)
      if (tid < nk) rk[tid] = 0u;
      __syncthreads();
      keff = nk < K ? nk : K;
      if (nk > 0) {
        const int parts = kBT / nk, j = tid % nk, part = tid / nk;
        if (part < parts) {
          const int q0 = part * nk / parts, q1 = (part + 1) * nk / parts;
          const uint64_t kj = cand[j];
          uint32_t c = 0u;
          int q = q0;
          for (; q + 8 <= q1; q += 8) {  // (eight reads in flight)
            uint64_t t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) t[u] = cand[q + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) c += t[u] > kj ? 1u : 0u;
          }
          for (; q < q1; ++q) c += cand[q] > kj ? 1u : 0u;
          if (c) atomicAdd(&rk[j], c);
        }
        __syncthreads();
        if (tid < nk && rk[tid] < (uint32_t)keff) emit_row((int)rk[tid], cand[tid]);
      }
    } else if (!raise && K <= NW && nk <= 2 * kBT) {
      // The list alone, at most two keys a lane: each wave's K best by K
      // rounds of the wave's maximum (taken out of the lane that holds it),
      // then wave 0 takes the best K of the waves' the same way.
      const int wid = tid / kWave;
      uint64_t k0 = 0ull, k1 = 0ull, best = 0ull;  // best: on lane i, the wave's i-th
      if (tid < nk) k0 = key_of(kid[tid], true_bits(kid[tid], kx[tid]));
      if (tid + kBT < nk) k1 = key_of(kid[tid + kBT], true_bits(kid[tid + kBT], kx[tid + kBT]));
      for (int i = 0; i < K; ++i) {
        const uint64_t m = wave_max_u64_uni(k0 > k1 ? k0 : k1);
        if (m == 0ull) break;
        if (lane == i) best = m;
        if (k0 == m) k0 = 0ull;
        else if (k1 == m) k1 = 0ull;
      }
      if (lane < K) cand[wid * K + lane] = best;
      __syncthreads();
      keff = nk < K ? nk : K;
      if (wid == 0) {
        uint64_t c[NW * 16 / kWave];  // (NW * K <= 256 keys, four a lane)
#pragma unroll
        for (int u = 0; u < NW * 16 / kWave; ++u)
          c[u] = lane + u * kWave < NW * K ? cand[lane + u * kWave] : 0ull;
        uint64_t top = 0ull;
        for (int i = 0; i < keff; ++i) {
          uint64_t mine = 0ull;
#pragma unroll
          for (int u = 0; u < NW * 16 / kWave; ++u) mine = c[u] > mine ? c[u] : mine;
          const uint64_t m = wave_max_u64_uni(mine);
          if (lane == i) top = m;
#pragma unroll
          for (int u = 0; u < NW * 16 / kWave; ++u)
            if (c[u] == m) c[u] = 0ull;
        }
        if (lane < keff) emit_row(lane, top);
      }
    } else if (!raise) {  // the list alone, ranked on chip
      keff = select_top(
          K, [&](auto &&f) { for (int i = tid; i < nk; i += kBT) f(key_of(kid[i], true_bits(kid[i], kx[i]))); },
          emit_row, hist, cand, ss, true);
    } else {  // and the seen ids below the bound, which the penalty raises
      keff = select_top(
          K,
          [&](auto &&f) {
            for (int i = tid; i < nk; i += kBT) f(key_of(kid[i], true_bits(kid[i], kx[i])));
            for (int w = tid; w < mw; w += kBT) {
              uint32_t bits = seen[w] & ~kill[w];
              while (bits) {
                const int v = w * 32 + __ffs(bits) - 1;
                bits &= bits - 1u;
                const float x =
                    bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(rowp)[v] << 16)
                         : reinterpret_cast<const float *>(rowp)[v];
                if (!(x >= xthr)) f(key_of(v, true_bits(v, x)));
              }
            }
          },
          emit_row, hist, cand, ss, true);
    }
  } else {
    // A lower bound of the row's K-th key: the K-th largest key of a sample,
    // every lane's first 16-byte chunk.  Only keys at or above it can be
    // among the row's best K, so the row's select counts those alone (0: the
    // sample is smaller than K and bounds nothing).
    __shared__ uint64_t t0_s;
    if (tid == 0) t0_s = 0ull;
    const int ns = select_top(
        K,
        [&](auto &&f) {
          if (tid < NGs)
            for (int j = 0; j < epc; ++j) {
              const int v = tid * epc + j;
              f(key_of(v, true_bits(v, elem(c0, j))));
            }
        },
        [&](int rank, uint64_t k) {
          if (rank == K - 1) t0_s = k;
        },
        hist, cand, ss);
    __syncthreads();
    const uint64_t t0 = ns == K ? t0_s : 0ull;
    const uint32_t t0hi = (uint32_t)(t0 >> 32);
    // The row pass scores every id as plain; removal lowers a score and a
    // penalty p >= 1 lowers a log-probability (all <= 0), so an id whose
    // plain key misses the bound misses it truly, and the few that pass are
    // rescored.  A penalty p < 1 raises the seen ids' scores: those the row
    // pass dropped are scored again from the seen mask.
    const bool raise = s.rep < 1.0f;
    keff = select_top(
        K,
        [&](auto &&f) {
          visit_row(rowp, bf16, V, [&](int v, float x) {
            const uint32_t ob = plain_bits(x);
            if (ob >= t0hi) {
              uint64_t k = key_of(v, ob);
              if (k >= t0) {
                if (has_bit(kill, v) || (s.rep != 1.0f && has_bit(seen, v)))
                  k = key_of(v, true_bits(v, x));
                if (k >= t0) f(k);
              }
            }
          });
          if (raise)
            for (int w = tid; w < mw; w += kBT) {
              uint32_t bits = seen[w] & ~kill[w];
              while (bits) {
                const int v = w * 32 + __ffs(bits) - 1;
                bits &= bits - 1u;
                const float x =
                    bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(rowp)[v] << 16)
                         : reinterpret_cast<const float *>(rowp)[v];
                if (key_of(v, plain_bits(x)) < t0) {
                  const uint64_t k = key_of(v, true_bits(v, x));
                  if (k >= t0) f(k);
                }
              }
            }
        },
        emit_row, hist, cand, ss, true);
  }
  for (int i = keff + tid; i < K; i += kBT) keys_out[i] = 0ull;
}

__global__ __launch_bounds__(kBT, 1) void k_beam_merge(BeamArgs a) {
  extern __shared__ __align__(16) uint32_t bsm[];
  __shared__ SelShared ss;
  const int p = blockIdx.x, tid = threadIdx.x, V = a.s.V, K = a.width;
  const uint64_t *keys = a.row_keys + (int64_t)p * a.nb * K;
  uint32_t *hist = bsm;
  uint64_t *cand = reinterpret_cast<uint64_t *>(hist + kBeamSelBins);
  float *sc = a.out_scores + (int64_t)p * K;
  int32_t *bm = a.out_beams + (int64_t)p * K, *tk = a.out_tokens + (int64_t)p * K;
  const int64_t n = (int64_t)a.nb * K;
  const int keff = select_top(
      K, [&](auto &&f) { for (int64_t e = tid; e < n; e += kBT) f(keys[e]); },
      [&](int rank, uint64_t k) {
        const uint32_t e = 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu);
        sc[rank] = unordered32((uint32_t)(k >> 32));
        bm[rank] = (int32_t)(e / (uint32_t)V);
        tk[rank] = (int32_t)(e % (uint32_t)V);
      },
      hist, cand, ss, true);
  for (int i = keff + tid; i < K; i += kBT) {  // fewer candidates than slots
    sc[i] = -INFINITY;
    bm[i] = -1;
    tk[i] = -1;
  }
}

// k_beam_merge for a prompt whose num_beams * K row keys fit one wave, a key
// a lane: each key's rank is the count of larger keys, read lane by lane.
__global__ __launch_bounds__(kWave) void k_beam_merge_wave(BeamArgs a) {
  const int p = blockIdx.x, lane = threadIdx.x, V = a.s.V, K = a.width;
  const int n = a.nb * K;
  const uint64_t k = lane < n ? a.row_keys[(int64_t)p * n + lane] : 0ull;
  int rank = 0;
  for (int q = 0; q < kWave; ++q) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, q);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), q);
    rank += (((uint64_t)hi << 32) | lo) > k ? 1 : 0;
  }
  const int present = __popcll(__ballot(k != 0ull));
  const int keff = present < K ? present : K;
  float *sc = a.out_scores + (int64_t)p * K;
  int32_t *bm = a.out_beams + (int64_t)p * K, *tk = a.out_tokens + (int64_t)p * K;
  if (k != 0ull && rank < keff) {
    const uint32_t e = 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu);
    sc[rank] = unordered32((uint32_t)(k >> 32));
    bm[rank] = (int32_t)(e / (uint32_t)V);
    tk[rank] = (int32_t)(e % (uint32_t)V);
  }
  if (lane >= keff && lane < K) {  // fewer candidates than slots
    sc[lane] = -INFINITY;
    bm[lane] = -1;
    tk[lane] = -1;
  }
}

size_t beam_rows_lds(int32_t V) {
  const size_t mw = ((size_t)V + 31) / 32;
  // masks, radix bins, the select's keys, the sum pass's kept ids and logits
  return (((2 * mw + 3) & ~size_t(3)) + kBeamSelBins) * 4 + (size_t)kSelCap * 16;
}

hipError_t launch_beam(const BeamArgs &a, hipStream_t st) {
  if (a.s.B <= 0) return hipSuccess;
  const size_t lds = beam_rows_lds(a.s.V);
  const size_t mlds = (size_t)kBeamSelBins * 4 + (size_t)kSelCap * 8;
  static std::atomic<uint64_t> rows_set{0}, merge_set{0};  // devices where the limit is raised
  if (hipError_t e = ensure_dyn_lds(reinterpret_cast<const void *>(&k_beam_rows),
                                    (int)kSelectMaxDynLds, rows_set);
      e != hipSuccess)
    return e;
  if (hipError_t e = ensure_dyn_lds(reinterpret_cast<const void *>(&k_beam_merge),
                                    (int)kSelectMaxDynLds, merge_set);
      e != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_beam_rows, dim3(a.s.B), dim3(kBT), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((int64_t)a.nb * a.width <= kWave)
    hipLaunchKernelGGL(k_beam_merge_wave, dim3(a.s.B / a.nb), dim3(kWave), 0, st, a);
  else
    hipLaunchKernelGGL(k_beam_merge, dim3(a.s.B / a.nb), dim3(kBT), mlds, st, a);
  return hipGetLastError();
}

}  // namespace tsel
