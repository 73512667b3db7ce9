// k_res.hip -- sampling without top_k at temperature 1 over a row that stays
// in registers, for gfx950.
//
// One 1024-thread workgroup per row; the row (up to 16 chunks of 16 bytes per
// lane) arrives with eight chunks in flight per lane.  The history, the static
// masks and the on-chip list offsets are staged in LDS while the first chunks
// fly, behind barriers that order LDS only, so nothing waits for the row
// before it is needed.  Each chunk, as it lands, loses its removed ids (-inf),
// hands the penalized scores of its seen ids to the on-chip list and adds its
// masses to the exact mass histogram (reference: the maximum of every lane's
// first chunk, plus 2).  Then:
//
//  * cumulative bin masses name the bin of the top_p boundary and the bin of
//    the draw;
//  * in a bf16 row a bin whose score interval holds a single bf16 value is a
//    tie group (plus a few list elements): the boundary or the draw inside it
//    follows by arithmetic on the group's equal masses, and one pass over the
//    registers counts group members in id order to name the id;
//  * any other bin is collected (key, mass) into LDS and ordered there;
//  * a bin that fits neither way falls back to a bisection over selection
//    keys that re-reads the row.
//
// Sources: "Transmuter.Generation (transmuter v2.0.0)", module doc (the
// processors and warpers, in order; temperature, top_k and top_p are the
// sampling warpers) and the inverse-CDF draw of a caller uniform over the
// kept ids in (score desc, id asc) order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "k_res_common.hpp"

namespace tsel {
namespace {

using namespace res;
// Elements that may share a mass bin with another value are kept on chip
// as they land, so that such a bin is ordered from that buffer without
// another pass over the row.  In a bf16 row these are the scores below
// 2^(7 - bin_mant) in magnitude: with 2^bin_mant bins per binade a bin spans
// less than 2^-bin_mant in score, and above that magnitude the bf16 spacing
// is at least as wide, so a bin there holds one value at most.  In a
// binary32 row, the scores within kHeadDelta nats of the first chunks'
// maximum.
constexpr float kHeadDelta = 3.0f;
constexpr int kHeadCap = 512;  // head elements kept on chip

struct ResShared {
  BinView view;
  WalkResult walk[2];
  uint32_t klim[2];
  // id-rank tasks
  float gv[2];
  int gk[2];
  int gi[2], gw[2], gr[2];
  int gid[2];
  int wtot[2][NW][16];
  int n_ind_all;
  int ltie;
};

// Ordered score key of the smallest score whose mass falls in bin >= b.
__device__ __forceinline__ uint32_t bin_floor_key(int b, int nb, int shift, int base, float cref) {
  if (b <= 0) return 0u;
  if (b >= nb) return 0xFFFFFFFFu;
  uint32_t lo = ordered_f32(-INFINITY), hi = ordered_f32(INFINITY);
  while (hi - lo > 1) {
    const uint32_t mid = lo + (hi - lo) / 2;
    if (mass_bin(__float_as_uint(mass_of<false>(unordered_f32(mid), 0.0f, cref)), shift, base,
                 nb) >= b)
      hi = mid;
    else
      lo = mid;
  }
  return hi;
}

// The same key found by one whole wave: a first guess from the logarithm of
// the bin's smallest mass, then three 64-way searches that narrow a window
// of 2^16 keys around it to one key.  The map from score to bin is monotone
// (the device exp2 is), so the window holds the edge whenever its two ends
// fall on either side; otherwise one lane bisects the whole key range.
// Every lane of the wave calls; all get the key.
__device__ __forceinline__ uint32_t bin_floor_key_wave(int b, int nb, int shift, int base,
                                                       float cref) {
  if (b <= 0) return 0u;
  if (b >= nb) return 0xFFFFFFFFu;
  const int lane = threadIdx.x & (kWave - 1);
  auto in_bin = [&](uint32_t k) {
    return mass_bin(__float_as_uint(mass_of<false>(unordered_f32(k), 0.0f, cref)), shift, base, nb) >= b;
  };
  const float e_lo = __uint_as_float((uint32_t)(b + base) << shift);
  // y with y log2(e) - cref = log2(e_lo)
  const double y0 = ((double)__log2f(e_lo) + (double)cref) / 1.4426950408889634;
  const uint32_t k0 = ordered_f32((float)y0);
  uint32_t lo = k0 > 0x8000u ? k0 - 0x8000u : 1u;          // in_bin(lo) must be false
  uint32_t hi = k0 < 0xFFFF7FFFu ? k0 + 0x8000u : 0xFFFFFFFEu;  // in_bin(hi) must be true
  const bool ok = !in_bin(lo) && in_bin(hi);
  if (ok) {
    // invariant: !in_bin(lo), in_bin(hi)
    for (int r = 0; r < 3 && hi - lo > 1; ++r) {
      const uint64_t step = ((uint64_t)(hi - lo) + 63) / 64;
      const uint64_t kk = (uint64_t)lo + (uint64_t)(lane + 1) * step;  // no wrap in 64 bits
      const bool pass = kk >= (uint64_t)hi || in_bin((uint32_t)kk);
      const uint64_t m = __ballot(pass);  // lanes from the first passing one on pass
      const int first = __ffsll((long long)m) - 1;  // lane 63 always passes (kk >= hi)
      const uint32_t new_hi = (uint32_t)min((uint64_t)hi, (uint64_t)lo + (uint64_t)(first + 1) * step);
      const uint32_t new_lo = (uint32_t)((uint64_t)lo + (uint64_t)first * step);
      lo = new_lo;
      hi = new_hi;
    }
    if (hi - lo <= 1) return hi;
  }
  // fall back: one lane bisects the whole range
  uint32_t r = 0u;
  if (lane == 0) r = bin_floor_key(b, nb, shift, base, cref);
  return (uint32_t)__shfl((int)r, 0, kWave);
}

// The bf16 value set inside scores [klo, khi) (ordered keys): returns the
// number of bf16 values there, capped at 2, and the first one.
__device__ __forceinline__ int bf16_values_in(uint32_t klo, uint32_t khi, float *first) {
  if (klo >= khi) return 0;
  float f = unordered_f32(klo);
  uint32_t u = __float_as_uint(f);
  if (u & 0xFFFFu) u = (f > 0.0f) ? (u & 0xFFFF0000u) + 0x10000u : (u & 0xFFFF0000u);
  float v1 = __uint_as_float(u);
  if (v1 == 0.0f) v1 = 0.0f;  // -0 is +0
  if (ordered_f32(v1) >= khi) return 0;
  *first = v1;
  const uint32_t b1 = __float_as_uint(v1);
  const uint32_t b2 = (v1 >= 0.0f) ? b1 + 0x10000u : b1 - 0x10000u;
  const float v2 = __uint_as_float(b2);
  return ordered_f32(v2) >= khi ? 1 : 2;
}

// Killed elements of a chunk become -inf; the per-word masks come from the
// kill bits by bit-field sign extension (no table read: an LDS read here
// would wait behind the histogram adds of the chunk before).
template <int DT>
__device__ __forceinline__ uint4 kill_alu(uint4 c, uint32_t kb) {
  uint32_t w[4] = {c.x, c.y, c.z, c.w};
  const uint32_t ninf = Elem<DT>::kNegInf;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t m;
    if (DT == 1) {
      const uint32_t lo = (uint32_t)((int32_t)(kb << (31 - 2 * q)) >> 31) & 0x0000FFFFu;
      const uint32_t hi = (uint32_t)((int32_t)(kb << (30 - 2 * q)) >> 31) & 0xFFFF0000u;
      m = lo | hi;
    } else {
      m = (uint32_t)((int32_t)(kb << (31 - q)) >> 31);
    }
    w[q] = (m & ninf) | (~m & w[q]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

template <int DT, int R>
__global__ __launch_bounds__(NT, 1) void k_res(SelectArgs a) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  constexpr int PIPE = R < kPipe ? R : kPipe;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RowShared sh;
  __shared__ ResShared rs;
  const Lds s = carve(a, smem);
  uint16_t *woff = reinterpret_cast<uint16_t *>(smem + a.off_woff);
  const int tid = threadIdx.x, row = blockIdx.x, V = a.V;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const int NG = V / EPC;  // whole chunks (>= 1 on this path)
  const int glast = NG - 1;
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  // ---- 0. small loads first, then the row (none waits for another) -------
  Early ea;
  early_loads<DT>(a, row, rowp, ea);
  const int tail_n = V - NG * EPC;
  const uint32_t *tw = ea.tw;
  uint4 reg[R];
#pragma unroll
  for (int i = 0; i < PIPE; ++i) reg[i] = load16(rowp + (int64_t)min(tid + i * NT, glast) * 16);
  RowInfo ri;
  if (row_prologue(a, row, ri)) return;
  const int32_t *h = a.hist + (int64_t)row * a.hist_stride;

  // ---- 1. staging: masks, list, table (LDS only) ----------------------------
  uint64_t *hist = reinterpret_cast<uint64_t *>(s.area);
  const int nb = a.nb;
  const int shift = 23 - a.bin_mant;
  const int base = (127 - kBinBelow) << a.bin_mant;
  const uint32_t lowmask = (1u << shift) - 1u;
  // Two copies of the histogram, lanes of odd index adding to the second
  // (half the same-address collisions of one instruction); the second copy
  // starts 8 bytes further on so that the copies of a bin fall on different
  // banks.  After the row it is folded into the first and its space holds
  // the collect buffer.  Then the head buffer and the ordered sub-bin.
  uint64_t *hist2 = hist + nb + 1;
  uint64_t *hkey = reinterpret_cast<uint64_t *>(s.area + 16 * (size_t)nb + 16);
  float *hval = reinterpret_cast<float *>(hkey + kHeadCap);
  uint64_t *okey = reinterpret_cast<uint64_t *>(hval + kHeadCap);
  float *oval = reinterpret_cast<float *>(okey + kGatherCap);
  uint64_t *ckey = hist2;
  float *cval = reinterpret_cast<float *>(hist2 + a.ccap);
  stage_clear(s, sh, a.mw, 4 * a.mw, a.mw);
  for (int b = tid; b < nb; b += NT) hist[b] = 0ull;
  for (int b = tid; b < nb; b += NT) hist2[b] = 0ull;
  const int n_list = stage(a, row, ri, s, sh, h, ea, woff);
  if (n_list < 0) return;

  // ---- 2. chunks as they land: kill, list, histogram -------------------------
  float lmax = -INFINITY, ref = 0.0f, cref = 0.0f, thr = INFINITY;
  // (captured: |score| < 1.0625 * 2^(7 - bin_mant), which covers every bin
  // that reaches below 2^(7 - bin_mant), bins being narrower than the margin)
  const float kMultiZone = 1.0625f * __uint_as_float((uint32_t)(127 + 7 - a.bin_mant) << 23);
  // The chunk's kill bits, read one chunk ahead so that the read does not
  // queue behind the chunk's own histogram adds.  (Seen ids are killed here
  // too; their scores are gathered onto the list once the row has landed.)
  auto chunk_kill = [&](int i) {
    const int g = tid + i * NT;
    const bool ok = g < NG || (g == NG && tail_n > 0);
    return chunk_bits<DT>(s.kmask, ok ? g : 0);
  };
  uint32_t kb_n = chunk_kill(0);
  tail_words<DT>(ea, V);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i + PIPE < R) reg[i + PIPE] = load16(rowp + (int64_t)min(tid + (i + PIPE) * NT, glast) * 16);
    const int g = tid + i * NT;
    const uint32_t kb = kb_n;
    if (i + 1 < R) kb_n = chunk_kill(i + 1);
    uint4 c = launder(reg[i]);
    if (g == NG && tail_n > 0) c = make_uint4(tw[0], tw[1], tw[2], tw[3]);
    if (g < NG || (g == NG && tail_n > 0)) {
      c = kill_alu<DT>(c, kb);
    } else {
      c = make_uint4(E::kNegInf, E::kNegInf, E::kNegInf, E::kNegInf);
    }
    reg[i] = c;
    float cmax = E::get(c, 0);
#pragma unroll
    for (int j = 1; j < EPC; ++j) cmax = fmaxf(cmax, E::get(c, j));
    lmax = fmaxf(lmax, cmax);
    asm volatile("" : "+v"(lmax));  // the running maximum per chunk, not deferred
    if (i == 0) {
      const float m0 = block_max_f32_lds<NT>(lmax, sh.red_f32);
      ref = m0 == -INFINITY ? 0.0f : m0 + kRefSlack;
      cref = ref * kLog2e;
      thr = DT == 1 ? -kMultiZone : m0 - kHeadDelta;
    }
    if (DT == 1 ? cmax > -kMultiZone : cmax >= thr) {
      // the head of the row, as it lands (a chunk whose maximum is below it
      // holds none)
      uint32_t hb = 0u;
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const float x = E::get(c, j);
        hb |= ((DT == 1 ? fabsf(x) < kMultiZone : x >= thr) ? 1u : 0u) << j;
      }
      if (hb) {
#pragma unroll
        for (int j = 0; j < EPC; ++j)
          if ((hb >> j) & 1u) {
            const int slot = atomicAdd(&sh.n_coll, 1);
            if (slot < kHeadCap) hkey[slot] = sel_key(E::get(c, j), (uint32_t)(g * EPC + j));
          }
      }
    }
    uint64_t *hh = (lane & 1) ? hist2 : hist;
#pragma unroll
    for (int j = 0; j < EPC; ++j) {
      const uint32_t bits = __float_as_uint(mass_of<false>(E::get(c, j), 0.0f, cref));
      atomicAdd(&hh[mass_bin(bits, shift, base, nb)], (1ull << 40) | (bits & lowmask));
    }
  }
  __syncthreads();  // the row has landed (in the caches too)
  for (int k = tid; k < n_list; k += NT) {
    const float y = penalize(E::load1(rowp, s.list_id[k]), a.rep);
    s.list_val[k] = y;
    lmax = fmaxf(lmax, y);
    if (DT == 1 ? fabsf(y) < kMultiZone : y >= thr) {
      const int slot = atomicAdd(&sh.n_coll, 1);
      if (slot < kHeadCap) hkey[slot] = sel_key(y, (uint32_t)s.list_id[k]);
    }
    const uint32_t bits = __float_as_uint(mass_of<false>(y, 0.0f, cref));
    atomicAdd(&hist[mass_bin(bits, shift, base, nb)], (1ull << 40) | (bits & lowmask));
  }
  const float mx = block_max_f32<NT>(lmax, sh.red_f32);
  if (tid == 0) {
    sh.n_list = n_list;
    sh.dense_pen = 0;
  }
  uint64_t kcut = 0ull;
  int token = 0;
  if (mx == -INFINITY) {  // every id removed: id 0, nothing kept
    if (tid == 0) a.out_tokens[row] = 0;
    if (a.out_processed) res_processed<DT>(a, row, s, INFINITY, ~0ull, n_list);
    return;
  }
  if ((mx - ref) * kLog2e >= (float)(kBinAbove - 1)) {
    // the maximum outran the reference: histogram again against it
    ref = mx;
    cref = ref * kLog2e;
    __syncthreads();
    for (int b = tid; b < nb; b += NT) hist[b] = hist2[b] = 0ull;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint4 c = launder(reg[i]);
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const uint32_t bits = __float_as_uint(mass_of<false>(E::get(c, j), 0.0f, cref));
        atomicAdd(&hist[mass_bin(bits, shift, base, nb)], (1ull << 40) | (bits & lowmask));
      }
    }
    for (int k = tid; k < n_list; k += NT) {
      const uint32_t bits = __float_as_uint(mass_of<false>(s.list_val[k], 0.0f, cref));
      atomicAdd(&hist[mass_bin(bits, shift, base, nb)], (1ull << 40) | (bits & lowmask));
    }
  }
  __syncthreads();
  for (int b = tid; b < nb; b += NT) hist[b] += hist2[b];  // fold the second copy in
  __syncthreads();

  // ---- 3. cumulative bin masses ------------------------------------------------
  // Thread t owns bins [t*bpt, t*bpt + bpt); C(b) = mass of bins >= b.
  const int bpt = (nb + NT - 1) / NT;
  double part = 0.0;
  for (int q = 0; q < bpt; ++q) {
    const int b = tid * bpt + q;
    if (b < nb) part += bin_mass(hist[b], b, shift, base);
  }
  double incl;  // mass of bins owned by threads >= tid
  {
    double v = part;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double t = __shfl_down(v, o, kWave);
      if (lane + o < kWave) v += t;
    }
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
    sh.found = -1;
  }
  __syncthreads();
  const double W = uni(sh.wprime);
  const bool use_top_p = a.top_p < 1.0f;
  const double pw = (double)a.top_p * W;
  const double u = (double)a.uniforms[row];
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
  const int bp = uni(sh.bin_p);
  const double C_bp1 = bp >= 0 ? uni(sh.sbase) : 0.0;  // mass above the boundary bin
  // the draw target u W' lies in [u C(bp + 1), u C(bp)]
  const double t_lo = bp < 0 ? u * W : u * C_bp1;
  const double t_hi = bp < 0 ? u * W : u * (C_bp1 + bin_mass(hist[bp], bp, shift, base));
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
  const int shi = uni(sh.bin_hi);
  int slo = uni(sh.found);
  if (slo < 0 || (bp >= 0 && slo < bp)) slo = bp >= 0 ? bp : shi;

  // ---- 4. the boundary and the draw ------------------------------------------
  __shared__ uint64_t gkey[kGatherCap];
  __shared__ float gval[kGatherCap];

  // View of bin b (all threads): single-valued test and its list elements,
  // ordered by key into okey / oval.  Returns false when the bin has more
  // list elements than fit.
  auto view_bin = [&](int b) -> bool {
    if (wid < 2) {
      const uint32_t k = bin_floor_key_wave(b + wid, nb, shift, base, cref);
      if (lane == 0) rs.klim[wid] = k;
    }
    if (tid == 0) rs.n_ind_all = 0;
    __syncthreads();
    const uint32_t klo = uni(rs.klim[0]), khi = uni(rs.klim[1]);
    if (tid == 0) {
      float v = 0.0f;
      const int nv = DT == 1 ? bf16_values_in(klo, khi, &v) : 2;
      rs.view.single = nv <= 1;
      rs.view.v = nv == 1 ? v : NAN;
      rs.view.e = nv == 1 ? mass_of<false>(v, 0.0f, cref) : 0.0f;
    }
    __syncthreads();
    const float v = uni(rs.view.v);
    for (int k = tid; k < n_list; k += NT) {
      const float y = s.list_val[k];
      const uint32_t ky = ordered_f32(y);
      if (ky >= klo && ky < khi && !(y == v)) {
        const int slot = atomicAdd(&rs.n_ind_all, 1);
        if (slot < kGatherCap) {
          gkey[slot] = sel_key(y, (uint32_t)s.list_id[k]);
          gval[slot] = mass_of<false>(y, 0.0f, cref);
        }
      }
    }
    __syncthreads();
    const int ni = uni(rs.n_ind_all);
    if (ni > kGatherCap) return false;
    for (int i = tid; i < ni; i += NT) {
      const uint64_t ki = gkey[i];
      int r = 0;
      for (int j = 0; j < ni; ++j) r += gkey[j] > ki;
      okey[r] = ki;
      oval[r] = gval[i];
    }
    __syncthreads();
    if (tid == 0) {
      int na = 0;
      const uint32_t kv = ordered_f32(v);
      for (int q = 0; q < ni; ++q) na += (uint32_t)(okey[q] >> 32) > kv;
      rs.view.n_ind = ni;
      rs.view.n_above = rs.view.single ? na : ni;
      rs.view.n_group = (int)(hist[b] >> 40) - ni;
    }
    __syncthreads();
    return true;
  };

  bool fallback = false;
  double Wp = W;
  int cut_kind = kNone, draw_kind = kNone;
  int cut_pos = 0x7FFFFFFF;
  int bs = -1;
  double bs_start = 0.0;
  if (bp >= 0) {
    if (!view_bin(bp)) {
      fallback = true;
    } else if (uni(rs.view.single)) {
      if (tid == 0) rs.walk[0] = single_walk(true, C_bp1, pw, rs.view, okey, oval, 0x7FFFFFFF);
      __syncthreads();
      cut_kind = uni(rs.walk[0].kind);
      if (cut_kind == kFail) fallback = true;
      Wp = uni(rs.walk[0].acc);
      cut_pos = uni(rs.walk[0].pos);
      if (cut_kind == kInd) kcut = uni(rs.walk[0].key);
    } else {
      cut_kind = kCollect;
    }
  }
  const float bp_v = uni(rs.view.v);  // the boundary bin's value (single-valued bins)
  double target = u * Wp;
  // The draw's bin: the bin whose cumulative mass interval holds the target
  // (bp counts only its kept part); every thread checks its own bins.
  auto find_draw_bin = [&]() {
    if (tid == 0) {
      sh.bin_hi = -1;
      sh.sbase = -1.0;
    }
    __syncthreads();
    {
      double C = above_me;
      for (int q = bpt - 1; q >= 0; --q) {
        const int b = tid * bpt + q;
        if (b >= nb || b < 1) continue;
        const double m = (bp >= 0 && b == bp) ? (Wp - C_bp1) : bin_mass(hist[b], b, shift, base);
        if (m > 0.0 && C <= target && target < C + m) {
          sh.bin_hi = b;
          sh.sbase = C;
        }
        C += m;
      }
    }
    __syncthreads();
    bs = uni(sh.bin_hi);
    bs_start = uni(sh.sbase);
    if (bs < 0) {  // rounding left the target outside every bin
      bs = bp >= 0 ? bp : slo;
      bs_start = -1.0;
    }
  };
  if (!fallback && cut_kind != kCollect) {
    find_draw_bin();
    if (bs_start < 0.0) {
      fallback = true;
    } else if (bs == bp && bp >= 0) {
      // same bin as the boundary: the view is still in place
      if (tid == 0) rs.walk[1] = single_walk(false, bs_start, target, rs.view, okey, oval, cut_pos);
      __syncthreads();
      draw_kind = uni(rs.walk[1].kind);
    } else if (!view_bin(bs)) {
      fallback = true;
    } else if (uni(rs.view.single)) {
      if (tid == 0) rs.walk[1] = single_walk(false, bs_start, target, rs.view, okey, oval, 0x7FFFFFFF);
      __syncthreads();
      draw_kind = uni(rs.walk[1].kind);
    } else {
      draw_kind = kCollect;
    }
    if (draw_kind == kFail) fallback = true;
  }
  const float bs_v = uni(rs.view.v);

  // ---- 5. one pass over the registers: tie-group ranks and collection --------
  // Group tasks: task 0 = the boundary's group member, task 1 = the draw's.
  const bool g0 = !fallback && cut_kind == kGroup;
  const bool g1 = !fallback && draw_kind == kGroup;
  // Collection: the boundary bin and the candidate draw bins when the
  // boundary bin is not single-valued; else the draw bin alone.
  int c_lo0 = 0, c_hi0 = -1, c_lo1 = 0, c_hi1 = -1;  // bin ranges to collect
  if (!fallback && cut_kind == kCollect) {
    c_lo0 = bp; c_hi0 = bp;
    c_lo1 = slo; c_hi1 = shi;
    uint32_t ncount = (uint32_t)(hist[bp] >> 40);
    if (shi >= 0)
      for (int b = slo; b <= shi; ++b)
        if (b != bp) ncount += (uint32_t)(hist[b] >> 40);
    if (!(shi >= 1 && slo >= 1 && slo <= shi) || ncount > (uint32_t)a.ccap) fallback = true;
  } else if (!fallback && draw_kind == kCollect) {
    c_lo0 = bs; c_hi0 = bs;
    if ((uint32_t)(hist[bs] >> 40) > (uint32_t)a.ccap) fallback = true;
  }
  const bool collect = !fallback && (cut_kind == kCollect || draw_kind == kCollect);
  if (collect) {
    if (wid < 4) {
      const int bsel = wid == 0 ? c_lo0 : wid == 1 ? c_hi0 + 1 : wid == 2 ? c_lo1 : c_hi1 + 1;
      uint32_t r = 0u;
      if (wid < 2 || c_hi1 >= c_lo1) r = bin_floor_key_wave(bsel, nb, shift, base, cref);
      if (lane == 0) gkey[wid] = r;
    }
    __syncthreads();
  }
  // score limits of the collect intervals (a key of ~0 is +inf)
  float f0lo = INFINITY, f0hi = -INFINITY, f1lo = INFINITY, f1hi = -INFINITY;
  if (collect) {
    auto kf = [](uint32_t k) { return k == 0xFFFFFFFFu ? INFINITY : unordered_f32(k); };
    f0lo = kf(uni((uint32_t)gkey[0]));
    f0hi = kf(uni((uint32_t)gkey[1]));
    if (c_hi1 >= c_lo1) {
      f1lo = kf(uni((uint32_t)gkey[2]));
      f1hi = kf(uni((uint32_t)gkey[3]));
    }
  }
  // Intervals inside the head: their elements are already on chip.
  const int n_head = uni(sh.n_coll);
  // (bf16: the head holds every score in (-2, 2); binary32: every score >= thr)
  auto in_head = [&](float lo, float hi) {
    return DT == 1 ? (lo >= -kMultiZone && hi <= kMultiZone) : lo >= thr;
  };
  const bool from_head = collect && n_head <= kHeadCap && in_head(f0lo, f0hi) &&
                         (c_hi1 < c_lo1 || in_head(f1lo, f1hi));
  __syncthreads();  // every wave has read the head count before it may be reset
  if (from_head) {
    for (int k = tid; k < n_head; k += NT) hval[k] = mass_of<false>(key_score(hkey[k]), 0.0f, cref);
    ckey = hkey;  // the collected set is the head
    cval = hval;
  } else if (collect) {
    if (tid == 0) sh.n_coll = 0;
  }
  __syncthreads();
  const bool col_pass = collect && !from_head;
  bool ltie_all = false;
  uint32_t tmask = 0u;       // chunks of this thread holding list elements of a group
  float v0 = NAN, v1 = NAN;  // group values (NaN: idle task, no element equals it)
  if (g0 || g1) {
    if (tid == 0) {
      rs.gv[0] = bp_v; rs.gk[0] = g0 ? rs.walk[0].rank + 1 : 0;
      rs.gv[1] = bs_v; rs.gk[1] = g1 ? rs.walk[1].rank + 1 : 0;
      rs.gi[0] = rs.gi[1] = -1;
      rs.gid[0] = rs.gid[1] = -1;
      rs.ltie = 0;
    }
    __syncthreads();
    v0 = g0 ? uni(rs.gv[0]) : NAN;
    v1 = g1 ? uni(rs.gv[1]) : NAN;
    // list elements equal to a group value join the group (rare): only then
    // does the count look them up chunk by chunk
    // which chunks of which thread hold such a list element: 16 bits per
    // thread, two threads a word, in the (now idle) ordered-view buffer
    uint32_t *tiew = reinterpret_cast<uint32_t *>(okey);
    for (int q = tid; q < NT / 2; q += NT) tiew[q] = 0u;
    __syncthreads();
    for (int k = tid; k < n_list; k += NT) {
      const float y = s.list_val[k];
      if (y == v0 || y == v1) {
        rs.ltie = 1;
        const int gg = s.list_id[k] / EPC, t = gg % NT, ci = gg / NT;
        atomicOr(&tiew[t >> 1], 1u << ((t & 1) * 16 + ci));
      }
    }
    __syncthreads();
    ltie_all = uni(rs.ltie) != 0;
    tmask = (tiew[tid >> 1] >> ((tid & 1) * 16)) & 0xFFFFu;
  }
  // One pass over the registers: members per (wave, chunk index) of the tie
  // groups by wave-wide ballots, and the elements of the collect intervals
  // with their keys and masses.
  auto pass = [&](auto cnt_tag, auto col_tag) {
    constexpr bool CNT = decltype(cnt_tag)::value, COL = decltype(col_tag)::value;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint4 c = launder(reg[i]);
      const int g = tid + i * NT;
      int t0 = 0, t1 = 0;
      uint32_t mb = 0u;
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const float x = E::get(c, j);
        if (CNT) {
          t0 += __popcll(__ballot(x == v0));
          t1 += __popcll(__ballot(x == v1));
        }
        if (COL) mb |= (((x >= f0lo && x < f0hi) || (x >= f1lo && x < f1hi)) ? 1u : 0u) << j;
      }
      if (CNT) {
        if (ltie_all) {
          int l0 = 0, l1 = 0;
          if ((tmask >> i) & 1u) {
            uint32_t bits = chunk_bits<DT>(s.smask, g);
            while (bits) {
              const int j = __ffs(bits) - 1;
              bits &= bits - 1;
              const float y = s.list_val[list_slot(g * EPC + j, s.smask, woff)];
              l0 += y == v0;
              l1 += y == v1;
            }
          }
          if (__ballot(l0 != 0) != 0ull) t0 += wave_sum_i32(l0);
          if (__ballot(l1 != 0) != 0ull) t1 += wave_sum_i32(l1);
        }
        if (lane == 0) {
          rs.wtot[0][wid][i] = t0;
          rs.wtot[1][wid][i] = t1;
        }
      }
      if (COL) {
        if (mb) {
#pragma unroll
          for (int j = 0; j < EPC; ++j)
            if ((mb >> j) & 1u) {
              const float x = E::get(c, j);
              const int slot = atomicAdd(&sh.n_coll, 1);
              if (slot < a.ccap) {
                ckey[slot] = sel_key(x, (uint32_t)(g * EPC + j));
                cval[slot] = mass_of<false>(x, 0.0f, cref);
              }
            }
        }
      }
    }
  };
  using T1 = std::integral_constant<bool, true>;
  using T0 = std::integral_constant<bool, false>;
  if ((g0 || g1) && col_pass) pass(T1{}, T1{});
  else if (g0 || g1) pass(T1{}, T0{});
  else if (col_pass) pass(T0{}, T1{});
  if (col_pass) {
    for (int k = tid; k < n_list; k += NT) {
      const float y = s.list_val[k];
      if ((y >= f0lo && y < f0hi) || (y >= f1lo && y < f1hi)) {
        const int slot = atomicAdd(&sh.n_coll, 1);
        if (slot < a.ccap) {
          ckey[slot] = sel_key(y, (uint32_t)s.list_id[k]);
          cval[slot] = mass_of<false>(y, 0.0f, cref);
        }
      }
    }
  }
  __syncthreads();
    if (g0 || g1) {
      // chunk index and wave of the k-th member in id order (chunk index,
      // then thread, then element)
      if (tid < 32) {
        const int t = tid >> 4, i = tid & 15;
        const bool on = (t == 0 ? g0 : g1) && i < R;
        int T = 0;
        if (on)
          for (int w = 0; w < NW; ++w) T += rs.wtot[t][w][i];
        // inclusive scan over the 16 lanes of this task
        int inc = T;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const int y = __shfl_up(inc, o, 16);
          if (i >= o) inc += y;
        }
        const int k = on ? rs.gk[t] : 0;
        if (on && inc - T < k && k <= inc) {
          int rem = k - (inc - T), w = 0;
          while (w < NW - 1 && rs.wtot[t][w][i] < rem) { rem -= rs.wtot[t][w][i]; ++w; }
          rs.gi[t] = i;
          rs.gw[t] = w;
          rs.gr[t] = rem;
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (!(t == 0 ? g0 : g1)) continue;
        const int ii = rs.gi[t];
        if (ii < 0) { fallback = true; continue; }
        if (wid == rs.gw[t]) {
          const int g = tid + ii * NT;
          const float vv = rs.gv[t];
          // members among this lane's elements of chunk ii (every chunk is
          // tested with a constant index: selecting reg[ii] would become a
          // run-time index and send the whole row through scratch memory)
          uint32_t mbits = 0u;
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const uint4 c = launder(reg[i]);
            uint32_t b = 0u;
#pragma unroll
            for (int j = 0; j < EPC; ++j) b |= (E::get(c, j) == vv ? 1u : 0u) << j;
            mbits = i == ii ? b : mbits;
          }
          if (ltie_all && ((tmask >> ii) & 1u)) {
            uint32_t bits = chunk_bits<DT>(s.smask, g);
            while (bits) {
              const int j = __ffs(bits) - 1;
              bits &= bits - 1;
              if (s.list_val[list_slot(g * EPC + j, s.smask, woff)] == vv) mbits |= 1u << j;
            }
          }
          const int cnt = __popc(mbits);
          const int inc = wave_incl_scan_i32(cnt);
          const int rem = rs.gr[t];
          if (inc - cnt < rem && rem <= inc) {
            int r = rem - (inc - cnt);
            uint32_t bits = mbits;
            int j = 0;
            while (bits) {
              j = __ffs(bits) - 1;
              bits &= bits - 1;
              if (--r == 0) break;
            }
            rs.gid[t] = g * EPC + j;
          }
        }
        __syncthreads();
      }
    }
  if ((g0 && rs.gid[0] < 0) || (g1 && rs.gid[1] < 0)) fallback = true;
  if (!fallback && g0) kcut = sel_key(bp_v, (uint32_t)rs.gid[0]);
  if (!fallback && draw_kind == kGroup) token = rs.gid[1];
  if (!fallback && draw_kind == kInd) token = (int)key_index(rs.walk[1].key);

  // ---- 6. collected bins: exact order on chip --------------------------------
  if (collect && !fallback) {
    const int nc = min(sh.n_coll, a.ccap);
    __shared__ uint64_t subh[256];
    __shared__ double sub_start;
    __shared__ int sub_sel, n_g;
    const int sshift = shift - 8;
    const uint32_t slowmask = (1u << sshift) - 1u;
    // Elements of bin bsel with key >= kmin, after the mass `start`: a
    // sub-histogram over the next 8 mass bits finds the sub-bin where the
    // running mass crosses `goal`; that sub-bin is ordered by key.  Returns
    // the selected key (cut: the last kept; draw: the drawn), or 0 when the
    // sub-bin is too large to order.
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
        const double inc = wave_incl_scan_f64(lane_sum);
        double before = start + (inc - lane_sum);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const double after = before + m[q];
          const bool hit = cut ? (before < goal && goal <= after) : (before <= goal && goal < after);
          if (hit && m[q] > 0.0) { sub_sel = 255 - 4 * tid - q; sub_start = before; }
          before = after;
        }
      }
      __syncthreads();
      if (sub_sel < 0) {
        // nothing crossed inside the bin (rounding at its end): its lowest
        // non-empty sub-bin
        if (tid == 0) {
          double before = start;
          int lowest = -1;
          for (int sb = 255; sb >= 0; --sb) {
            const uint64_t acc_w = subh[sb];
            const uint64_t cnt = acc_w >> 40;
            if (!cnt) continue;
            if (lowest >= 0) {
              const uint32_t lo_bits = ((uint32_t)(bsel + base) << shift) | ((uint32_t)lowest << sshift);
              const int expo = (int)(lo_bits >> 23);
              const double ulp = __longlong_as_double((long long)(expo - 150 + 1023) << 52);
              const uint64_t pw_ = subh[lowest];
              before += (double)(pw_ >> 40) * (double)__uint_as_float(lo_bits) +
                        (double)(pw_ & ((1ull << 40) - 1)) * ulp;
            }
            lowest = sb;
          }
          sub_sel = lowest;
          sub_start = before;
        }
        __syncthreads();
      }
      const int ss = sub_sel;
      if (ss < 0) return 0ull;
      for (int i = tid; i < nc; i += NT) {
        const uint32_t bits = __float_as_uint(cval[i]);
        if (mass_bin(bits, shift, base, nb) == bsel && ckey[i] >= kmin &&
            (int)((bits >> sshift) & 255u) == ss) {
          const int slot = atomicAdd(&n_g, 1);
          if (slot < kGatherCap) { gkey[slot] = ckey[i]; gval[slot] = cval[i]; }
        }
      }
      __syncthreads();
      const int ng = n_g;
      if (ng > kGatherCap) return 0ull;
      for (int i = tid; i < ng; i += NT) {
        const uint64_t ki = gkey[i];
        int r = 0;
        for (int j = 0; j < ng; ++j) r += gkey[j] > ki;
        okey[r] = ki;
        oval[r] = gval[i];
      }
      __syncthreads();
      // walk in key order: 64 lanes, four elements each
      if (tid < kWave) {
        double m[4], lsum = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = 4 * tid + q;
          m[q] = j < ng ? (double)oval[j] : 0.0;
          lsum += m[q];
        }
        const double inc = wave_incl_scan_f64(lsum);
        double A = sub_start + (inc - lsum);
        int sel = -1;
        double a_sel = 0.0;  // cut: mass before the first removed element
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = 4 * tid + q;
          if (j < ng && sel < 0) {
            if (cut) {
              if (A >= goal) { sel = j; a_sel = A; }  // first removed
            } else if (A + m[q] > goal) {
              sel = j;                                // drawn
            }
          }
          if (sel < 0) A += m[q];
        }
        // first lane with a hit
        const uint64_t hits = __ballot(sel >= 0);
        const int first = hits ? __ffsll((long long)hits) - 1 : -1;
        const int fsel = __shfl(sel, first < 0 ? 0 : first, kWave);
        const double fa = __shfl(a_sel, first < 0 ? 0 : first, kWave);
        const double total = __shfl(inc, kWave - 1, kWave);
        if (tid == 0) {
          int pick;
          double through;
          if (cut) {
            pick = first < 0 ? ng - 1 : fsel - 1;  // last kept
            through = first < 0 ? sub_start + total : fa;
            if (pick < 0) { pick = 0; through = sub_start + (double)oval[0]; }
          } else {
            pick = first < 0 ? ng - 1 : fsel;
            through = 0.0;
          }
          sh.kcut = okey[pick];
          sh.wprime = through;
        }
      }
      __syncthreads();
      *acc = sh.wprime;
      return sh.kcut;
    };
    if (cut_kind == kCollect) {
      double acc = 0.0;
      kcut = resolve(bp, 0ull, C_bp1, pw, true, &acc);
      if (kcut == 0ull) {
        fallback = true;
      } else {
        Wp = acc;
        target = u * Wp;
        find_draw_bin();
        if (bs_start < 0.0) {
          fallback = true;
        } else if (bs == bp || (bs >= slo && bs <= shi)) {
          double d;
          const uint64_t tk = resolve(bs, bs == bp ? kcut : 0ull, bs_start, target, false, &d);
          if (tk == 0ull || tk < kcut) fallback = true;
          else token = (int)key_index(tk);
        } else {
          fallback = true;
        }
      }
    } else {
      double d;
      const uint64_t tk = resolve(bs, 0ull, bs_start, target, false, &d);
      if (tk == 0ull) fallback = true;
      else token = (int)key_index(tk);
    }
  }
  if (fallback) token = bisect_select<DT, true>(a, row, s, sh, -INFINITY, cref, &kcut);
  if (tid == 0) a.out_tokens[row] = token;
  if (a.out_processed) res_processed<DT>(a, row, s, -INFINITY, kcut, n_list);
}

template <int DT, int R>
static hipError_t launch_res_t(const SelectArgs &a, size_t lds, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};  // devices where the limit is raised
  const void *fn = reinterpret_cast<const void *>(&k_res<DT, R>);
  if (hipError_t e = ensure_dyn_lds(fn, (int)kSelectMaxDynLds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL((k_res<DT, R>), dim3(a.B), dim3(NT), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_res(const SelectArgs &a, int res, size_t lds, hipStream_t st) {
  if (a.dtype == 1) {
    if (res == 16) return launch_res_t<1, 16>(a, lds, st);
    if (res == 8) return launch_res_t<1, 8>(a, lds, st);
    return launch_res_t<1, 4>(a, lds, st);
  }
  if (res == 16) return launch_res_t<0, 16>(a, lds, st);
  if (res == 8) return launch_res_t<0, 8>(a, lds, st);
  return launch_res_t<0, 4>(a, lds, st);
}

}  // namespace tsel
