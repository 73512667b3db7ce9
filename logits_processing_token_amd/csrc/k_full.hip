// k_full.hip -- sampling on gfx950: k_topk for a top_k (a running threshold
// filters each row into an on-chip candidate buffer; temperature, top_k,
// top_p and the draw then run exactly on the candidates), and k_full for
// rows without top_k or whose ties overflow that buffer (k_topk then runs
// the full path in the same workgroup).
//
// One 1024-thread workgroup per row.  The row stays in registers when it
// fits (16 chunks of 16 bytes per lane: 131072 bf16 or 65536 binary32 ids);
// its loads are issued first and fly while the history is staged.  Then:
//
//  1. Mass histogram.  Every score y gets the mass e = 2^((y - r) log2 e)
//     relative to a reference r just above the first chunk's maximum.  The
//     binary32 bits of e name a bin (exponent and top mantissa bits), and one
//     64-bit LDS add per element accumulates (count << 40) + (the mantissa
//     bits below the bin's top bits).  Each bin's mass then follows exactly:
//     every element of the bin shares the exponent and top bits, so the sum
//     of their e is (count * (2^23 + top bits) + low-bit sum) * 2^(E-150).
//     The order of the adds does not matter and nothing is rounded.
//  2. The bin of the top_p boundary and the bins that can hold the sample
//     (a short range) follow from the cumulative bin masses.
//  3. The elements of those bins are collected (a bin edge maps back to a
//     score threshold because the hardware exp2 is monotone, which a GPU test
//     checks exhaustively), ordered by (score desc, id asc) and walked with
//     binary64 prefix sums: the last kept id of top_p, the kept mass W' and
//     the id whose cumulative mass first exceeds u * W'.
//
// A reference too far below the row maximum moves to the maximum (a second
// histogram pass); bins too large to collect, and rows whose history needs
// the in-stream penalty, use a bisection over selection keys that re-reads
// the row.  Sources: "Transmuter.Generation (transmuter v2.0.0)", module doc
// (temperature, top_k, top_p are the sampling warpers, in that order), and
// the inverse-CDF draw of a caller uniform in (score desc, id asc) order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k_mass.hpp"
#include "k_vkey.hpp"

namespace tsel {

// ---------------------------------------------------------------------------
// The histogram pass over a streamed bf16 row, by value.  Equal bf16 scores
// have equal masses, so the row is counted into one bin per bf16 value (a
// 32-bit LDS add per element, two copies by lane parity; no temperature
// division and no exponential per element) and each value bin then adds
// count * (its mass's word) to the mass histogram: the same exact words as
// one add per element.  The value bins span the keys [klo, klo + kVBins - 1)
// with klo the lowest key whose mass reaches mass bin 1 (lower keys count for
// nothing, as in the mass histogram).  Elements that a value bin cannot
// stand for take the mass histogram one by one: near-zero scores (one key
// for a range of values), keys past the value bins, scores penalized in the
// stream, and the list.  With `keep`, elements of mass bins >= keep_bin are
// appended to the collect buffer; a value-counted one as its raw score and
// id, marked by a negative mass, to be finished after the pass.  Returns
// this lane's maximum final score.
template <bool TOPK>
__device__ __forceinline__ float value_hist_pass(const SelectArgs &a, int row, const Lds &s,
                                                 RowShared &sh, float t_y, float c, bool keep,
                                                 int keep_bin, uint64_t *hist, uint64_t *ckey,
                                                 float *cval, uint32_t *vb) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int nb = a.nb, shift = 23 - a.bin_mant, base = (127 - kBinBelow) << a.bin_mant;
  const uint32_t lowmask = (1u << shift) - 1u;
  const float T = TOPK ? a.temperature : 1.0f;
  const int NG = a.V / 8;
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  const bool dense_pen = sh.dense_pen != 0;
  auto final_y = [&](float x) { return (T != 1.0f) ? x / T : x; };
  auto bin_of = [&](float y) {
    return mass_bin(__float_as_uint(mass_of<TOPK>(y, t_y, c)), shift, base, nb);
  };
  // Smallest key whose value reaches mass bin `target` (the near-zero keys
  // stand for -2^-kZoneExp and +2^-kZoneExp; neither is counted by value).
  auto first_key = [&](int target) {
    auto val = [&](uint32_t k) {
      const float z = __uint_as_float((uint32_t)(127 - kZoneExp) << 23);
      return k == kKeyZoneNeg ? -z : k == kKeyZonePos ? z : vkey_value(k);
    };
    uint32_t lo = kKeyLowFinite - 1u, hi = vkey(0x7F80u);  // -inf: no mass; +inf: every bin
    while (hi - lo > 1u) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      if (bin_of(final_y(val(mid))) >= target) hi = mid;
      else lo = mid;
    }
    return hi;
  };
  __shared__ uint32_t lim[2];
  if (tid == 0) lim[0] = first_key(1);
  if (tid == kWave) lim[1] = keep ? first_key(keep_bin) : 0xFFFFFFFFu;
  for (int i = tid; i < 2 * kVStride; i += NT) vb[i] = 0u;
  __syncthreads();
  const uint32_t klo = lim[0], kkeep = lim[1];
  const uint32_t khi = klo + (uint32_t)(kVBins - 1);  // keys from here: one by one
  uint32_t *vbl = vb + (lane & 1) * kVStride;
  float lmx = -INFINITY;
  uint32_t kmx = 0u;  // the largest key of the row's elements (of this lane)
  // An element that a value bin does not stand for (few per row: near-zero
  // scores, keys past the bins, scores penalized in the stream): one by one
  // into the mass histogram, appended when kept.
  auto one_by_one = [&](int v, uint32_t raw, bool pen) {
    float x = __uint_as_float(raw << 16);
    if (pen) x = penalize(x, a.rep);
    const float y = final_y(x);
    lmx = fmaxf(lmx, y);
    const uint32_t bits = __float_as_uint(mass_of<TOPK>(y, t_y, c));
    const int b = mass_bin(bits, shift, base, nb);
    atomicAdd(&hist[b], (1ull << 40) | (bits & lowmask));
    if (keep && b >= keep_bin) {
      const int slot = atomicAdd(&sh.n_coll, 1);
      if (slot < a.ccap) {
        ckey[slot] = sel_key(y, (uint32_t)v);
        cval[slot] = __uint_as_float(bits);
      }
    }
  };
  // One chunk (every lane of the wave calls; `real`: the chunk is in the
  // row).  Killed elements become -inf, below every bin.  Every element adds
  // 1 to the bin of its value key clamped to the bins: keys below klo to bin
  // 0 (no mass), keys from khi on to a spare word past the bins, the two
  // near-zero keys to their own words, which the conversion skips.  The
  // elements a value bin does not stand for (near-zero, past the bins,
  // penalized in the stream) go one by one, a penalized one first taking its
  // count back.  Returns the elements to keep by value (bit j for element
  // j).  (Chunks past the row read as +0: near-zero, and not real.)
  const uint8_t *kbyte = reinterpret_cast<const uint8_t *>(s.kmask);
  const uint8_t *sbyte = reinterpret_cast<const uint8_t *>(s.smask);
  const uint32_t klo1 = klo - 1u, ninf = 0xFF80FF80u;
  auto bin_word = [&](uint32_t k) { return &vbl[min(max(k, klo1), khi) - klo1]; };
  auto chunk = [&](int g, uint4 cw, uint32_t kb, uint32_t sb, bool real) -> uint32_t {
    cw = vkill(cw, kb, ninf);
    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
    uint32_t slow = 0u, kept = 0u, kc = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t t;
      const uint32_t k = vkey_t((j & 1) ? w[j >> 1] >> 16 : w[j >> 1], t);
      atomicAdd(bin_word(k), 1u);
      slow |= (t == 0u || k >= khi) ? 1u << j : 0u;
      kept |= k >= kkeep ? 1u << j : 0u;
      kc = max(kc, k);
    }
    if (sb) {  // (the penalized elements' raw keys do not count)
      kc = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t t;
        const uint32_t k = vkey_t((j & 1) ? w[j >> 1] >> 16 : w[j >> 1], t);
        kc = ((sb >> j) & 1u) ? kc : max(kc, k);
      }
    }
    kmx = real ? max(kmx, kc) : kmx;
    slow = real ? slow | sb : 0u;
    kept = real ? kept & ~slow : 0u;
    if (slow) {
#pragma unroll 1
      for (uint32_t m = slow; m; m &= m - 1u) {
        const int j = __ffs(m) - 1;
        const uint32_t raw = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const bool pen = (sb >> j) & 1u;
        if (pen) {
          uint32_t t;
          atomicSub(bin_word(vkey_t(raw, t)), 1u);
        }
        one_by_one(g * 8 + j, raw, pen);
      }
    }
    return kept;
  };
  // The stream: batches of U chunks through a buffer resource (a read past
  // the row returns 0 and touches no memory, so every load is issued by every
  // lane and the batches alternate between two register sets: each batch's
  // loads fly while the other is counted).  Each chunk's kill (and
  // stream-penalty) byte is read one chunk ahead.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(rowp), (short)0, NG * 16, 0x00020000);
  auto ld = [&](int g) {
    const u32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(rs, g * 16, 0, 0);
    return make_uint4(q.x, q.y, q.z, q.w);
  };
  uint32_t kb_n = tid < NG ? kbyte[tid] : 0u;
  uint32_t sb_n = dense_pen && tid < NG ? sbyte[tid] : 0u;
  // A batch's kept elements are appended as raw score and id at slots that
  // one add per wave and batch reserves (a wave scan of the lanes' counts
  // places them).
  auto batch = [&](int i, const uint4 *cw) {  // batch i: chunks tid + (i U + u) NT
    uint32_t km[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = tid + (i * U + u) * NT;
      km[u] = 0u;
      if (__ballot(g < NG) == 0ull) continue;  // (past the row for the whole wave)
      const uint32_t kb = kb_n, sb = sb_n;
      const int gn = min(g + NT, NG - 1);
      kb_n = kbyte[gn];
      sb_n = dense_pen ? sbyte[gn] : 0u;
      km[u] = chunk(g, cw[u], kb, sb, g < NG);
    }
    if (keep) {
      int n = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) n += __popc(km[u]);
      const int incl = wave_incl_scan_i32(n);
      const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
      if (tot > 0) {
        int first = 0;
        if (lane == kWave - 1) first = atomicAdd(&sh.n_coll, tot);
        int o = __builtin_amdgcn_readlane(first, kWave - 1) + incl - n;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int g = tid + (i * U + u) * NT;
          const uint32_t w[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
#pragma unroll 1
          for (uint32_t m = km[u]; m; m &= m - 1u, ++o) {
            const int j = __ffs(m) - 1;
            if (o < a.ccap) {
              ckey[o] = ((uint64_t)((w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu) << 32) | (uint32_t)(g * 8 + j);
              cval[o] = -1.0f;
            }
          }
        }
      }
    }
  };
  const int nbat = (NG + NT * U - 1) / (NT * U);
  uint4 ca[U], cb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) ca[u] = ld(tid + u * NT);
  for (int i = 0; i < nbat; i += 2) {
#pragma unroll
    for (int u = 0; u < U; ++u) cb[u] = ld(tid + ((i + 1) * U + u) * NT);
    batch(i, ca);
#pragma unroll
    for (int u = 0; u < U; ++u) ca[u] = ld(tid + ((i + 2) * U + u) * NT);
    if (i + 1 < nbat) batch(i + 1, cb);
  }
  // the list: penalized seen ids and the row's tail, one by one
  const int n_list = sh.n_list;
  for (int i = tid; i < n_list; i += NT) {
    const float y = final_y(s.list_val[i]);
    lmx = fmaxf(lmx, y);
    const uint32_t bits = __float_as_uint(mass_of<TOPK>(y, t_y, c));
    const int b = mass_bin(bits, shift, base, nb);
    atomicAdd(&hist[b], (1ull << 40) | (bits & lowmask));
    if (keep && b >= keep_bin) {
      const int slot = atomicAdd(&sh.n_coll, 1);
      if (slot < a.ccap) {
        ckey[slot] = sel_key(y, (uint32_t)s.list_id[i]);
        cval[slot] = __uint_as_float(bits);
      }
    }
  }
  __syncthreads();
  // value bins -> mass histogram (bin 0: below klo, nothing; the near-zero
  // keys' words: elements counted one by one)
  for (int b = 1 + tid; b < kVBins; b += NT) {
    const uint32_t n = vb[b] + vb[kVStride + b];
    const uint32_t kb = klo + (uint32_t)b - 1u;
    if (n == 0u || kb == kKeyZoneNeg || kb == kKeyZonePos) continue;
    const uint32_t bits = __float_as_uint(mass_of<TOPK>(final_y(vkey_value(kb)), t_y, c));
    atomicAdd(&hist[mass_bin(bits, shift, base, nb)],
              (uint64_t)n * ((1ull << 40) | (bits & lowmask)));
  }
  // the kept value-counted elements: their keys and masses
  if (keep) {
    const int nc = min(sh.n_coll, a.ccap);
    for (int i = tid; i < nc; i += NT) {
      if (cval[i] < 0.0f) {
        const uint64_t kk = ckey[i];
        const float y = final_y(__uint_as_float((uint32_t)(kk >> 32) << 16));
        ckey[i] = sel_key(y, (uint32_t)kk);
        cval[i] = mass_of<TOPK>(y, t_y, c);
      }
    }
  }
  // The largest key stands for its value unless it is a near-zero key: then
  // every element of the lane lies at or below that key's range, and those
  // in it went one by one.
  const bool kval = kmx >= kKeyLowFinite && kmx != kKeyZoneNeg && kmx != kKeyZonePos;
  return fmaxf(lmx, kval ? final_y(vkey_value(kmx)) : -INFINITY);
}

// ---------------------------------------------------------------------------
// Histogram, bins, collect and walk for one row.  visit(f) calls f(id, y)
// once for every element of the row (dense stream and list), y the final
// score before top_k / top_p (killed ids as -inf).  Returns the token, or -1
// when the bisection must decide; *kcut / *t_out describe the kept set.
//
// VF: the histogram pass counts a streamed bf16 row by value
// (value_hist_pass); a second pass, when the maximum outruns the reference,
// is the plain one.  keep1 (with VF): that pass also keeps every element of
// the mass bins from kKeepBelow binades under the reference up; when those
// bins hold the boundary's and the sample's and the buffer did not overflow,
// step 3 takes them from there instead of visiting the row again.
template <bool TOPK, bool VF = false, class Visit>
__device__ __forceinline__ int full_core(const SelectArgs &a, int row, const Lds &s,
                                         RowShared &sh, float t_y, float m0, Visit &&visit,
                                         uint64_t *kcut_out, float *t_out, float *cref_out,
                                         bool keep1 = false) {
  const int tid = threadIdx.x;
  const int nb = a.nb;
  const int shift = 23 - a.bin_mant;
  const int base = (127 - kBinBelow) << a.bin_mant;
  const uint32_t lowmask = (1u << shift) - 1u;
  uint64_t *hist = reinterpret_cast<uint64_t *>(s.area);
  uint64_t *ckey = reinterpret_cast<uint64_t *>(s.area + 8 * (size_t)nb);
  float *cval = reinterpret_cast<float *>(s.area + 8 * (size_t)nb + 8 * (size_t)a.ccap);

  // ---- 1. mass histogram (a second pass when the maximum outruns r) ----
  float ref = m0 == -INFINITY ? 0.0f : m0 + kRefSlack;
  float mx = -INFINITY;
  const int keep_bin = (kBinBelow - kKeepBelow) << a.bin_mant;  // first kept bin
  bool kept = false;  // the collect buffer holds every element of bins >= keep_bin
  for (int attempt = 0; attempt < 2; ++attempt) {
    const float c = ref * kLog2e;
    const bool vpass = VF && attempt == 0 && a.vbins != 0;  // (the value bins fit on chip)
    const bool keep = vpass && keep1;
    for (int i = tid; i < nb; i += NT) hist[i] = 0ull;
    if (tid == 0) sh.n_coll = 0;
    __syncthreads();
    float lmx = -INFINITY;
    if (vpass) {
      uint32_t *vb = reinterpret_cast<uint32_t *>(s.area + 8 * (size_t)nb + 12 * (size_t)a.ccap +
                                                  12 * (size_t)kGatherCap);
      lmx = value_hist_pass<TOPK>(a, row, s, sh, t_y, c, keep, keep_bin, hist, ckey, cval, vb);
    } else visit([&](int, float y) {
      lmx = fmaxf(lmx, y);
      const uint32_t bits = __float_as_uint(mass_of<TOPK>(y, t_y, c));
      atomicAdd(&hist[mass_bin(bits, shift, base, nb)], (1ull << 40) | (bits & lowmask));
    });
    mx = block_max_f32<NT>(lmx, sh.red_f32);
    kept = keep && sh.n_coll <= a.ccap;
    // Masses below 2^(kBinAbove - 1) stay under the top bin.
    if (mx == -INFINITY || (mx - ref) * kLog2e < (float)(kBinAbove - 1)) break;
    ref = mx;
    kept = false;
  }
  const float cref = ref * kLog2e;
  *cref_out = cref;
  *t_out = t_y;
  *kcut_out = 0ull;
  if (mx == -INFINITY || mx < t_y) {  // every id removed: id 0
    *kcut_out = ~0ull;
    *t_out = INFINITY;
    return 0;
  }
  // ---- 2. cumulative masses from the top bin down ------------------------
  // Thread t owns bins [t*bpt, t*bpt + bpt); C(b) = mass of bins >= b.
  const int bpt = (nb + NT - 1) / NT;
  double part = 0.0;
  for (int q = 0; q < bpt; ++q) {
    const int b = tid * bpt + q;
    if (b < nb) part += bin_mass(hist[b], b, shift, base);
  }
  double incl;  // mass of bins owned by threads >= tid
  {
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    double v = part;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double t = __shfl_down(v, o, kWave);
      if (lane + o < kWave) v += t;
    }
    __syncthreads();
    if (lane == 0) sh.red_f64[wid] = v;
    __syncthreads();
    double after = 0.0;
    for (int q = wid + 1; q < NW; ++q) after += sh.red_f64[q];
    incl = v + after;
  }
  const double above_me = incl - part;
  if (tid == 0) {
    sh.wprime = incl;
    sh.bin_p = -1;
    sh.bin_hi = -1;
  }
  __syncthreads();
  const double W = sh.wprime;
  const bool use_top_p = a.top_p < 1.0f;
  const double pw = (double)a.top_p * W;
  const double u = (double)a.uniforms[row];
  // top_p boundary bin bp: C(bp + 1) < pW <= C(bp)
  {
    double C = above_me;
    for (int q = bpt - 1; q >= 0; --q) {
      const int b = tid * bpt + q;
      if (b >= nb) continue;
      const double Cb1 = C;
      C += bin_mass(hist[b], b, shift, base);
      if (use_top_p && Cb1 < pw && C >= pw) { sh.bin_p = b; sh.sbase = Cb1; }
    }
  }
  __syncthreads();
  const int bp = sh.bin_p;
  const double C_bp1 = bp >= 0 ? sh.sbase : 0.0;  // C(bp + 1): mass above the boundary bin
  // W' lies in [C(bp + 1), C(bp)], so the target u W' lies in [t_lo, t_hi];
  // the sample's bin is between the bins holding t_hi and t_lo.
  const double t_lo = bp < 0 ? u * W : u * C_bp1;
  const double t_hi = bp < 0 ? u * W : u * (C_bp1 + bin_mass(hist[bp], bp, shift, base));
  if (tid == 0) {
    sh.bin_hi = -1;
    sh.found = -1;
  }
  __syncthreads();
  {
    double C = above_me;
    for (int q = bpt - 1; q >= 0; --q) {
      const int b = tid * bpt + q;
      if (b >= nb) continue;
      const double Cb1 = C;
      C += bin_mass(hist[b], b, shift, base);
      if (Cb1 <= t_lo && t_lo < C) { sh.bin_hi = b; sh.sbase = Cb1; }
      if (Cb1 <= t_hi && t_hi < C) sh.found = b;
    }
  }
  __syncthreads();
  const int shi = sh.bin_hi;                    // highest bin that can hold the sample
  const double S_top = shi >= 0 ? sh.sbase : 0.0;  // C(shi + 1)
  int slo = sh.found;                           // lowest bin that can hold the sample
  if (slo < 0 || (bp >= 0 && slo < bp)) slo = bp >= 0 ? bp : shi;
  uint32_t ncount = 0;
  if (shi >= 0)
    for (int b = slo; b <= shi; ++b) ncount += (uint32_t)(hist[b] >> 40);
  if (bp >= 0 && bp < slo) ncount += (uint32_t)(hist[bp] >> 40);
  if (!(shi >= 1 && slo >= 1 && slo <= shi && ncount <= (uint32_t)a.ccap)) return -1;

  // ---- 3. collect bin bp and bins [slo, shi] ----------------------------
  // Kept by the histogram pass when every bin needed lies at or above the
  // kept bins: the buffer then holds each of their elements (and others,
  // which step 4 filters out by bin).  Otherwise: bins are score intervals,
  // Y(b) = smallest ordered score key of bin >= b (four bisections run on
  // four lanes), and the row is visited again.
  if (!(kept && slo >= keep_bin && (bp < 0 || bp >= keep_bin))) {
    __shared__ uint32_t ylim[4];
    if (tid < 4) {
      const int bsel = tid == 0 ? slo : tid == 1 ? shi + 1 : tid == 2 ? bp : bp + 1;
      uint32_t r = 0u;
      if (tid < 2 || bp >= 0) {
        if (bsel >= nb) {
          r = 0xFFFFFFFFu;
        } else {
          uint32_t lo = ordered_f32(-INFINITY), hi = ordered_f32(INFINITY);
          while (hi - lo > 1) {
            const uint32_t mid = lo + (hi - lo) / 2;
            if (mass_bin(__float_as_uint(mass_of<TOPK>(unordered_f32(mid), t_y, cref)), shift, base,
                         nb) >= bsel)
              hi = mid;
            else
              lo = mid;
          }
          r = hi;
        }
      }
      ylim[tid] = r;
    }
    if (tid == 0) sh.n_coll = 0;
    __syncthreads();
    const uint32_t s_lo = ylim[0], s_hi = ylim[1], p_lo = ylim[2], p_hi = ylim[3];
    visit([&](int v, float y) {
      const uint32_t ky = ordered_f32(y);
      if ((ky >= s_lo && ky < s_hi) || (ky >= p_lo && ky < p_hi)) {
        const int slot = atomicAdd(&sh.n_coll, 1);
        if (slot < a.ccap) {
          ckey[slot] = sel_key(y, (uint32_t)v);
          cval[slot] = mass_of<TOPK>(y, t_y, cref);
        }
      }
    });
    __syncthreads();
  }
  const int nc = min(sh.n_coll, a.ccap);

  // ---- 4. exact order inside one bin --------------------------------------
  // Among the collected elements of level-1 bin bsel with key >= kmin,
  // starting from the mass `start` of everything before them: a
  // sub-histogram over the next 8 mass bits (exact masses, as for the bins)
  // finds the sub-bin where the running mass crosses `goal`; only that
  // sub-bin is ordered by key.  cut: the first element whose mass before it
  // is >= goal is removed (returns the last kept index, *acc = mass through
  // it).  draw: the first element whose mass through it is > goal.
  // Returns the selected key, or 0 when the sub-bin is too large to order.
  __shared__ uint64_t subh[256];
  __shared__ uint64_t gkey[kGatherCap];
  __shared__ float gval[kGatherCap];
  __shared__ double sub_start;
  __shared__ int sub_sel, n_g;
  __shared__ uint32_t g_emin, g_emax;
  const int sshift = shift - 8;
  const uint32_t slowmask = (1u << sshift) - 1u;
  auto resolve = [&](int bsel, uint64_t kmin, double start, double goal, bool cut,
                     double *acc) -> uint64_t {
    for (int i = tid; i < 256; i += NT) subh[i] = 0ull;
    if (tid == 0) { n_g = 0; sub_sel = -1; }
    __syncthreads();
    for (int i = tid; i < nc; i += NT) {
      const uint32_t bits = __float_as_uint(cval[i]);
      if (mass_bin(bits, shift, base, nb) == bsel && ckey[i] >= kmin)
        atomicAdd(&subh[(bits >> sshift) & 255u], (1ull << 40) | (bits & slowmask));
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l holds sub-bins 255 - 4l .. 252 - 4l (descending mass)
      double m[4], lane_sum = 0.0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int sb = 255 - 4 * tid - q;
        const uint64_t acc_w = subh[sb];
        const uint64_t cnt = acc_w >> 40;
        const uint32_t lo_bits = ((uint32_t)(bsel + base) << shift) | ((uint32_t)sb << sshift);
        const int expo = (int)(lo_bits >> 23);
        const double ulp = __longlong_as_double((long long)(expo - 150 + 1023) << 52);
        m[q] = cnt ? (double)cnt * (double)__uint_as_float(lo_bits) +
                         (double)(acc_w & ((1ull << 40) - 1)) * ulp
                   : 0.0;
        lane_sum += m[q];
      }
      const double incl = wave_incl_scan_f64(lane_sum);
      double before = start + (incl - lane_sum);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double after = before + m[q];
        const bool hit = cut ? (before < goal && goal <= after) : (before <= goal && goal < after);
        if (hit && m[q] > 0.0) { sub_sel = 255 - 4 * tid - q; sub_start = before; }
        before = after;
      }
      // Nothing crossed inside this bin (rounding at its end): take the
      // lowest non-empty sub-bin.
      if (tid == kWave - 1) {
        // (written only if no lane hit; checked after the barrier)
      }
    }
    __syncthreads();
    if (sub_sel < 0) {
      if (tid < kWave) {
        int lowest = -1;
        for (int sb = tid; sb < 256; sb += kWave)
          if ((subh[sb] >> 40) != 0) lowest = lowest < 0 ? sb : min(lowest, sb);
        // wave min over lanes of `lowest` (ignoring -1)
        int v = lowest < 0 ? 0x7FFFFFFF : lowest;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
        if (tid == 0 && v != 0x7FFFFFFF) {
          double before = start;
          for (int sb = 255; sb > v; --sb) {
            const uint64_t acc_w = subh[sb];
            const uint64_t cnt = acc_w >> 40;
            if (!cnt) continue;
            const uint32_t lo_bits = ((uint32_t)(bsel + base) << shift) | ((uint32_t)sb << sshift);
            const int expo = (int)(lo_bits >> 23);
            const double ulp = __longlong_as_double((long long)(expo - 150 + 1023) << 52);
            before += (double)cnt * (double)__uint_as_float(lo_bits) +
                      (double)(acc_w & ((1ull << 40) - 1)) * ulp;
          }
          sub_sel = v;
          sub_start = before;
        }
      }
      __syncthreads();
    }
    const int ss = sub_sel;
    if (ss < 0) return 0ull;
    if (tid == 0) { g_emin = 0xFFFFFFFFu; g_emax = 0u; }
    __syncthreads();
    auto in_group = [&](int i) {
      const uint32_t bits = __float_as_uint(cval[i]);
      return mass_bin(bits, shift, base, nb) == bsel && ckey[i] >= kmin &&
             (int)((bits >> sshift) & 255u) == ss;
    };
    for (int i = tid; i < nc; i += NT) {
      if (in_group(i)) {
        const int slot = atomicAdd(&n_g, 1);
        if (slot < kGatherCap) { gkey[slot] = ckey[i]; gval[slot] = cval[i]; }
        atomicMin(&g_emin, __float_as_uint(cval[i]));  // masses are >= 0: bits order
        atomicMax(&g_emax, __float_as_uint(cval[i]));
      }
    }
    __syncthreads();
    const int ng = n_g;
    if (ng > kGatherCap) {
      // A large group of equal masses (tied scores, typically): the mass
      // before its j-th member in key order is sub_start + j e, so the member's
      // rank follows by arithmetic and a radix select over the 64-bit keys
      // names it.  Unequal masses: the caller bisects.
      if (g_emin != g_emax) return 0ull;
      const double e = (double)__uint_as_float(g_emin);
      long long r;  // rank (0 = largest key) of the selected member
      double through;
      {
        const double q = (goal - sub_start) / e;
        if (cut) {  // first removed: smallest j with sub_start + j e >= goal
          long long j = (long long)ceil(q);
          if (j < 0) j = 0;
          while (j > 0 && sub_start + (double)(j - 1) * e >= goal) --j;
          while (j < ng && sub_start + (double)j * e < goal) ++j;
          r = (j < ng ? j : ng) - 1;  // last kept
          if (r < 0) r = 0;
        } else {    // smallest j with sub_start + (j + 1) e > goal
          long long j = (long long)floor(q);
          if (j < 0) j = 0;
          while (j > 0 && sub_start + (double)j * e > goal) --j;
          while (j < ng - 1 && sub_start + (double)(j + 1) * e <= goal) ++j;
          r = j < ng ? j : ng - 1;
        }
        through = sub_start + (double)(r + 1) * e;
      }
      const int k = (int)r + 1;
      // k-th largest key of the group: high words first, then low words.
      const uint32_t hiw = radix_kth_largest(
          [&](auto &&f) {
            for (int i = tid; i < nc; i += NT)
              if (in_group(i)) f((uint32_t)(ckey[i] >> 32));
          },
          k, s.rhist, sh);
      int above = 0;
      for (int i = tid; i < nc; i += NT)
        if (in_group(i) && (uint32_t)(ckey[i] >> 32) > hiw) ++above;
      above = block_sum_i32<NT>(above, sh.red_i32);
      const uint32_t low = radix_kth_largest(
          [&](auto &&f) {
            for (int i = tid; i < nc; i += NT)
              if (in_group(i) && (uint32_t)(ckey[i] >> 32) == hiw) f((uint32_t)ckey[i]);
          },
          k - above, s.rhist, sh);
      *acc = through;
      return ((uint64_t)hiw << 32) | low;
    }
    // rank order (keys are distinct), into the collect buffer's head
    // ordered copy: the scratch after the collect buffer
    uint64_t *okey = reinterpret_cast<uint64_t *>(s.area + 8 * (size_t)nb + 12 * (size_t)a.ccap);
    float *oval = reinterpret_cast<float *>(okey + kGatherCap);
    for (int i = tid; i < ng; i += NT) {
      const uint64_t ki = gkey[i];
      int r = 0;
      for (int j = 0; j < ng; ++j) r += gkey[j] > ki;
      okey[r] = ki;
      oval[r] = gval[i];
    }
    __syncthreads();
    if (tid == 0) {
      double A = sub_start;
      int sel = -1;
      if (cut) {
        for (int j = 0; j < ng; ++j) {
          if (A >= goal) break;
          A += (double)oval[j];
          sel = j;
        }
      } else {
        for (int j = 0; j < ng; ++j) {
          A += (double)oval[j];
          sel = j;
          if (A > goal) break;
        }
      }
      sh.kcut = sel >= 0 ? okey[sel] : 0ull;
      sh.wprime = A;
    }
    __syncthreads();
    *acc = sh.wprime;
    return sh.kcut;
  };

  uint64_t kc = 0ull;
  double Wp = W;
  if (bp >= 0) {
    kc = resolve(bp, 0ull, C_bp1, pw, true, &Wp);
    if (kc == 0ull) return -1;
  }
  // The sample's bin: walk bins from shi down (their masses; bp counts only
  // its kept part).
  const double target = u * Wp;
  if (tid == 0) {
    double C = S_top;
    int bs = -1;
    double before = S_top;
    for (int b = shi; b >= slo && b >= 1; --b) {
      const double mb = (bp >= 0 && b == bp) ? (Wp - C) : bin_mass(hist[b], b, shift, base);
      if (mb > 0.0 && C <= target && target < C + mb) { bs = b; before = C; break; }
      C += mb;
    }
    if (bs < 0) { bs = bp >= 0 ? bp : slo; before = -1.0; }
    sh.bin_hi = bs;
    sh.sbase = before;
  }
  __syncthreads();
  const int bs = sh.bin_hi;
  const double bs_start = sh.sbase;
  if (bs_start < 0.0) return -1;  // rounding left the target outside: bisect
  double dummy;
  const uint64_t tk = resolve(bs, bs == bp ? kc : 0ull, bs_start, target, false, &dummy);
  if (tk == 0ull || tk < kc) return -1;
  *kcut_out = kc;
  return (int)key_index(tk);
}

// ---------------------------------------------------------------------------
// The whole selection of one row by the full path; smem holds the on-chip
// layout of `a`.  Every thread of the workgroup calls.
template <int DT, int RES, bool SIMPLE>
__device__ __forceinline__ void full_row(const SelectArgs &a, int row, unsigned char *smem,
                                         RowShared &sh) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  constexpr int R = RES > 0 ? RES : 1;
  const Lds s = carve(a, smem);
  const int tid = threadIdx.x, V = a.V;
  const int NG = V / EPC;
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  const float T = SIMPLE ? 1.0f : a.temperature;  // SIMPLE: no temperature, no top_k
  const int k_eff = (!SIMPLE && a.top_k > 0) ? min(a.top_k, V) : 0;
  // Rows without top_k keep the row in registers when it fits; the loads fly
  // while the history is staged.
  const bool want_res = SIMPLE && RES > 0 && NG <= RES * NT;
  uint4 reg[R];
  if (want_res) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int g = tid + i * NT;
      if (g < NG) reg[i] = load16(rowp + (int64_t)g * 16);
    }
  }
  RowInfo ri;
  if (row_prologue(a, row, ri)) return;
  stage_row<DT>(a, row, ri, s, sh, !want_res);
  const bool dense_pen = sh.dense_pen != 0;
  const int n_list = sh.n_list;
  uint64_t kcut = 0ull;
  float t_out = -INFINITY, cref = 0.0f;
  int token;
  float t_y = -INFINITY;
  if (want_res && !dense_pen) {
    // ---- resident row ----
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int g = tid + i * NT;
      if (g < NG) reg[i] = kill_chunk<DT>(reg[i], g, s);
    }
    float m0 = -INFINITY;  // reference: the first chunk of every lane and the list
    if (tid < NG)
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const float x = E::get(reg[0], j);
        m0 = fmaxf(m0, (T != 1.0f) ? x / T : x);
      }
    for (int i = tid; i < n_list; i += NT) {
      const float x = s.list_val[i];
      m0 = fmaxf(m0, (T != 1.0f) ? x / T : x);
    }
    m0 = block_max_f32<NT>(m0, sh.red_f32);
    token = full_core<!SIMPLE>(a, row, s, sh, t_y, m0,
                      [&](auto &&f) {
                        // Each pass unpacks the resident words afresh: without
                        // this the compiler keeps the unpacked binary32 values
                        // of one pass for the next and spills them.
#pragma unroll
                        for (int i = 0; i < R; ++i)
                          asm volatile("" : "+v"(reg[i].x), "+v"(reg[i].y), "+v"(reg[i].z),
                                       "+v"(reg[i].w));
#pragma unroll
                        for (int i = 0; i < R; ++i) {
                          const int g = tid + i * NT;
                          if (g < NG)
#pragma unroll
                            for (int j = 0; j < EPC; ++j) {
                              const float x = E::get(reg[i], j);
                              f(g * EPC + j, (T != 1.0f) ? x / T : x);
                            }
                        }
                        for (int i = tid; i < n_list; i += NT) {
                          const float x = s.list_val[i];
                          f(s.list_id[i], (T != 1.0f) ? x / T : x);
                        }
                      },
                      &kcut, &t_out, &cref);
  } else {
    // ---- streamed row ----
    if (k_eff > 0) t_y = topk_threshold_stream<DT>(a, row, s, sh, k_eff);
    auto visit = [&](auto &&f) {
      stream_row<DT>(a, rowp, s, dense_pen,
                     [&](int v, float x) { f(v, (T != 1.0f) ? x / T : x); });
      for (int i = tid; i < n_list; i += NT) {
        const float x = s.list_val[i];
        f(s.list_id[i], (T != 1.0f) ? x / T : x);
      }
    };
    // reference: every lane's first chunk and the list, as the stream
    // transforms them (the histogram pass moves it up if the row's maximum
    // outruns it); a pass over the row when none of them is kept
    float m0 = -INFINITY;
    if (tid < NG) {
      const uint4 ck = kill_chunk<DT>(load16(rowp + (int64_t)tid * 16), tid, s);
      const uint32_t sb = dense_pen ? chunk_bits<DT>(s.smask, tid) : 0u;
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        float x = E::get(ck, j);
        if ((sb >> j) & 1u) x = penalize(x, a.rep);
        const float y = (T != 1.0f) ? x / T : x;
        if (y >= t_y) m0 = fmaxf(m0, y);
      }
    }
    for (int i = tid; i < n_list; i += NT) {
      const float x = s.list_val[i];
      const float y = (T != 1.0f) ? x / T : x;
      if (y >= t_y) m0 = fmaxf(m0, y);
    }
    m0 = block_max_f32<NT>(m0, sh.red_f32);
    if (m0 == -INFINITY) {
      visit([&](int, float y) {
        if (y >= t_y) m0 = fmaxf(m0, y);
      });
      m0 = block_max_f32<NT>(m0, sh.red_f32);
    }
    token = full_core<!SIMPLE, DT == 1>(a, row, s, sh, t_y, m0, visit, &kcut, &t_out, &cref, true);
  }
  if (token < 0) token = bisect_select<DT>(a, row, s, sh, t_y, cref, &kcut);
  if (tid == 0) a.out_tokens[row] = token;
  if (a.out_logprobs) {
    const float lp = kept_logprob<DT>(a, row, s, sh, t_out, kcut, token);
    if (tid == 0) a.out_logprobs[row] = lp;
  }
  if (a.out_processed) write_processed<DT>(a, row, s, sh, t_out, kcut);
}

template <int DT, int RES, bool SIMPLE>
__global__ __launch_bounds__(NT, 1) void k_full(SelectArgs a, int pending_only) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RowShared sh;
  const int row = blockIdx.x;
  if (pending_only && a.out_tokens[row] != kPending) return;
  full_row<DT, RES, SIMPLE>(a, row, smem, sh);
}

// ---------------------------------------------------------------------------
template <int DT, int RES, bool SIMPLE>
static hipError_t launch_full_t(const SelectArgs &a, size_t lds, hipStream_t st, int pending) {
  static std::atomic<uint64_t> lds_set{0};  // devices where the limit is raised
  const void *fn = reinterpret_cast<const void *>(&k_full<DT, RES, SIMPLE>);
  if (hipError_t e = ensure_dyn_lds(fn, (int)kSelectMaxDynLds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL((k_full<DT, RES, SIMPLE>), dim3(a.B), dim3(NT), lds, st, a, pending);
  return hipGetLastError();
}

// simple: temperature 1 and no top_k (the row may stay in registers).
template <int DT>
static hipError_t launch_full_dt(const SelectArgs &a, int res, size_t lds, hipStream_t st,
                                 int pending, bool simple) {
  if (!simple) return launch_full_t<DT, 0, false>(a, lds, st, pending);
  if (res == 16) return launch_full_t<DT, 16, true>(a, lds, st, pending);
  if (res == 8) return launch_full_t<DT, 8, true>(a, lds, st, pending);
  if (res == 4) return launch_full_t<DT, 4, true>(a, lds, st, pending);
  return launch_full_t<DT, 0, true>(a, lds, st, pending);
}

hipError_t launch_full(const SelectArgs &a, int res, size_t lds, hipStream_t st, int pending) {
  const bool simple = a.temperature == 1.0f && a.top_k <= 0;
  return a.dtype == 1 ? launch_full_dt<1>(a, res, lds, st, pending, simple)
                      : launch_full_dt<0>(a, res, lds, st, pending, simple);
}

// =========================================================================
// k_topk: sampling with a top_k the candidate buffer holds.
// af: the same call with the full path's on-chip layout, which finishes a
// row whose ties overflow the buffer (smem holds the larger of the two).
template <int DT>
__global__ __launch_bounds__(NT, 1) void k_topk(SelectArgs a, SelectArgs af) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RowShared sh;
  const Lds s = carve(a, smem);
  const int tid = threadIdx.x, row = blockIdx.x, V = a.V;
  RowInfo ri;
  if (row_prologue(a, row, ri)) return;
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  const int NG = V / EPC;
  // every lane's first chunk and the stream's first batch fly while the
  // history is staged
  uint4 c0 = make_uint4(0u, 0u, 0u, 0u);
  if (tid < NG) c0 = load16(rowp + (int64_t)tid * 16);
  uint4 c[U], nx[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = NT + tid + u * NT;
    if (g < NG) c[u] = load16(rowp + (int64_t)g * 16);
  }
  stage_row<DT>(a, row, ri, s, sh);
  const bool dense_pen = sh.dense_pen != 0;
  const int n_list = sh.n_list;
  const float T = a.temperature;
  const int k_eff = min(a.top_k, V);
  const int tcap = a.tcap;
  float *cx = reinterpret_cast<float *>(s.area);
  int32_t *ci = reinterpret_cast<int32_t *>(s.area + 4 * tcap);
  if (tid == 0) {
    sh.count = 0;
    sh.overflow = 0;
  }
  __syncthreads();
  auto append = [&](int v, float x) {
    const int slot = atomicAdd(&sh.count, 1);
    if (slot < tcap) { cx[slot] = x; ci[slot] = v; }
    else sh.overflow = 1;
  };
  // element j of a chunk whose stream-penalty bits are sb (read once per
  // chunk: a read per element would wait behind the appends' LDS adds)
  auto prep = [&](const uint4 &c, uint32_t sb, int j) {
    float x = E::get(c, j);
    if ((sb >> j) & 1u) x = penalize(x, a.rep);
    return x;
  };
  auto pen_bits = [&](int g) { return dense_pen ? chunk_bits<DT>(s.smask, g) : 0u; };
  // Threshold from the first chunk of every lane: a lower bound of the k-th
  // largest alive score among them, hence of the row's.
  // (a coarse bound: a lower one only lets more candidates in; the
  // histogram borrows the candidate buffer, still empty: 24 tcap bytes)
  if (tid < NG) c0 = kill_chunk<DT>(c0, tid, s);
  const uint32_t sb0 = tid < NG ? pen_bits(tid) : 0u;
  const int nbins = 24 * tcap >= 16 * NT ? 4 * NT : NT;
  const float t0 = kth_lower_bound(
      [&](auto &&f) {
        if (tid < NG)
#pragma unroll
          for (int j = 0; j < EPC; ++j) {
            const float x = prep(c0, sb0, j);
            if (x > -INFINITY) f(x);
          }
      },
      k_eff, reinterpret_cast<uint32_t *>(s.area), nbins, sh);
  if (tid == 0) sh.tau_x = pre_temperature_floor(t0, T);
  __syncthreads();
  float flt = sh.tau_x;
  if (tid < NG)
#pragma unroll
    for (int j = 0; j < EPC; ++j) {
      const float x = prep(c0, sb0, j);
      if (x > -INFINITY && x >= flt) append(tid * EPC + j, x);
    }
  for (int i = tid; i < n_list; i += NT)
    if (s.list_val[i] >= flt) append(s.list_id[i], s.list_val[i]);
  __syncthreads();
  // Two batches of U chunks per lane: the next batch's loads fly while this
  // one is filtered (the barrier after it waits for LDS work only).
  for (int t0g = NT; t0g < NG && !sh.overflow; t0g += NT * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = t0g + NT * U + tid + u * NT;
      if (g < NG) nx[u] = load16(rowp + (int64_t)g * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = t0g + tid + u * NT;
      if (g < NG) {
        const uint4 ck = kill_chunk<DT>(c[u], g, s);
        const uint32_t sb = pen_bits(g);
#pragma unroll
        for (int j = 0; j < EPC; ++j) {
          const float x = prep(ck, sb, j);
          if (x > -INFINITY && x >= flt) append(g * EPC + j, x);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) c[u] = nx[u];
    lds_barrier();
    if (!sh.overflow && sh.count > tcap / 2) {
      // Prune: the new threshold is the k-th largest in the buffer.
      const int cnt = sh.count;
      const uint32_t tk = radix_kth_largest(
          [&](auto &&f) {
            for (int i = tid; i < cnt; i += NT) f(ordered_f32(cx[i]));
          },
          k_eff, s.rhist, sh);
      if (tid == 0)
        sh.tau_x = pre_temperature_floor(tk == 0u ? -INFINITY : unordered_f32(tk), T);
      __syncthreads();
      flt = sh.tau_x;
      constexpr int kPer = 8;  // tcap <= 8 * NT
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
        if (total > tcap / 2) sh.overflow = 1;  // ties fill the buffer
      }
      __syncthreads();
    }
  }
  __syncthreads();
  if (sh.overflow) {  // the full path takes this row, in this workgroup
    __syncthreads();
    full_row<DT, 0, false>(af, row, smem, sh);
    return;
  }
  // ---- exact temperature, top_k, top_p and draw on the candidates --------
  const int cnt = sh.count;
  for (int i = tid; i < cnt; i += NT) cx[i] = (T == 1.0f) ? cx[i] : cx[i] / T;
  __syncthreads();
  const uint32_t tk = radix_kth_largest(
      [&](auto &&f) {
        for (int i = tid; i < cnt; i += NT) f(ordered_f32(cx[i]));
      },
      k_eff, s.rhist, sh);
  const float t_y = tk == 0u ? -INFINITY : unordered_f32(tk);
  uint64_t *keys = reinterpret_cast<uint64_t *>(s.area + 8 * tcap);
  double *w = reinterpret_cast<double *>(s.area + 16 * tcap);
  if (tid == 0) sh.n_coll = 0;
  __syncthreads();
  for (int i = tid; i < cnt; i += NT)
    if (cx[i] >= t_y) keys[atomicAdd(&sh.n_coll, 1)] = sel_key(cx[i], (uint32_t)ci[i]);
  __syncthreads();
  const int nk = sh.n_coll;
  uint64_t kcut = 0ull;
  if (nk == 0) {  // every id removed
    if (tid == 0) {
      sh.token = 0;
      if (a.out_logprobs) a.out_logprobs[row] = lp_none();
    }
    kcut = ~0ull;
  } else {
    uint64_t *tmpk = reinterpret_cast<uint64_t *>(s.area);  // cx / ci are done
    for (int i = tid; i < nk; i += NT) {
      const uint64_t ki = keys[i];
      int r = 0;
      for (int j = 0; j < nk; ++j) r += keys[j] > ki;
      tmpk[r] = ki;
    }
    __syncthreads();
    for (int i = tid; i < nk; i += NT) keys[i] = tmpk[i];
    __syncthreads();
    const double m = (double)key_score(keys[0]);
    for (int i = tid; i < nk; i += NT) w[i] = exp((double)key_score(keys[i]) - m);
    __syncthreads();
    // The top_p cut and the draw by wave 0 over the ordered candidates, 64
    // at a time: binary64 prefix sums by row moves, a ballot naming the
    // first candidate that meets each condition.
    if (tid < kWave) {
      const int lane = tid;
      auto wv = [&](int j, int n) { return j < n ? w[j] : 0.0; };
      auto excl_of = [&](double incl, double carry) {  // the lane before's inclusive sum
        const double prev = __shfl_up(incl, 1, kWave);
        return lane == 0 ? carry : prev;
      };
      double W = 0.0;
      for (int b0 = 0; b0 < nk; b0 += kWave) W += wave_sum_f64(wv(b0 + lane, nk));
      // K: candidates are kept while the mass before them is below top_p of W
      int K = nk;
      double Wp = W;
      if (a.top_p < 1.0f) {
        const double p = (double)a.top_p;
        double carry = 0.0;
        for (int b0 = 0; b0 < nk; b0 += kWave) {
          const int j = b0 + lane;
          const double incl = carry + wave_incl_scan_f64_dpp(wv(j, nk));
          const double excl = excl_of(incl, carry);
          const uint64_t stop = __ballot(j < nk && !(excl / W < p));
          if (stop) {
            const int q = __ffsll((unsigned long long)stop) - 1;
            K = b0 + q;
            Wp = __shfl(excl, q, kWave);
            break;
          }
          carry = __shfl(incl, kWave - 1, kWave);
        }
      }
      // the draw: the first kept candidate whose mass through it exceeds u Wp
      const double target = (double)a.uniforms[row] * Wp;
      int pick = K - 1;
      double carry = 0.0;
      for (int b0 = 0; b0 < K; b0 += kWave) {
        const int j = b0 + lane;
        const double incl = carry + wave_incl_scan_f64_dpp(wv(j, K));
        const uint64_t hit = __ballot(j < K && incl > target);
        if (hit) {
          pick = b0 + __ffsll((unsigned long long)hit) - 1;
          break;
        }
        carry = __shfl(incl, kWave - 1, kWave);
      }
      if (lane == 0) {
        sh.token = (int)key_index(keys[pick]);
        sh.kcut = (K < nk) ? keys[K - 1] : 0ull;
        // the log-softmax of the kept scores at the token ("Log-probabilities")
        if (a.out_logprobs)
          a.out_logprobs[row] = (float)(((double)key_score(keys[pick]) - m) - log(Wp));
      }
    }
    __syncthreads();
    kcut = sh.kcut;
  }
  if (tid == 0) a.out_tokens[row] = sh.token;
  if (a.out_processed) write_processed<DT>(a, row, s, sh, nk == 0 ? INFINITY : t_y, kcut);
}

template <int DT>
static hipError_t launch_topk_t(const SelectArgs &a, const SelectArgs &af, size_t lds,
                                hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};  // devices where the limit is raised
  const void *fn = reinterpret_cast<const void *>(&k_topk<DT>);
  if (hipError_t e = ensure_dyn_lds(fn, (int)kSelectMaxDynLds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(k_topk<DT>, dim3(a.B), dim3(NT), lds, st, a, af);
  return hipGetLastError();
}

hipError_t launch_topk(const SelectArgs &a, const SelectArgs &af, size_t lds, hipStream_t st) {
  return a.dtype == 1 ? launch_topk_t<1>(a, af, lds, st) : launch_topk_t<0>(a, af, lds, st);
}

}  // namespace tsel
