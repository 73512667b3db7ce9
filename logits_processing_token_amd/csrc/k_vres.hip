// k_vres.hip -- sampling without top_k at temperature 1 over a bf16 row held
// in registers, with one histogram bin per bf16 value, for gfx950.
//
// One 1024-thread workgroup per row; the row (up to 16 chunks of 16 bytes per
// lane) arrives with four chunks in flight per lane, the first four asked
// for before the history and the masks are staged in LDS.  The seen ids'
// scores are gathered as their chunks arrive and penalized as they land.
// Each landed chunk loses its removed and seen ids (-inf) and is counted
// into a histogram whose bins are the bf16 values
// themselves: a score's bin is its ordered 16-bit pattern less an offset,
// worked out two scores at a time with packed 16-bit integer operations, so
// that the row costs no exponential and no float arithmetic per element.
// Lanes add into four copies of the histogram (fewer same-address
// collisions per instruction), folded once the row has landed.
//
//  * Bins start kDropNats below the maximum of every lane's first chunk:
//    lower scores weigh less than e^-kDropNats of the maximum each and count
//    for nothing.  Near zero the bf16 values are too dense for a bin each:
//    the scores of magnitude below 2^-kZoneExp share one bin, whose members
//    are listed one by one when it is not empty.
//  * Every other bin holds equal scores: its mass is its count times one
//    exponential, and its members tie, in id order.
//  * Individuals -- the seen ids with their penalized scores (any binary32
//    value) and the listed near-zero members -- each join the bin of the
//    largest bf16 value not above them and add their own mass there, as an
//    exact fixed-point sum.
//
// Cumulative bin masses then name the bin of the top_p boundary and the bin
// of the draw.  Inside a bin the order is: individuals above the bin's value
// (ordered on chip), the tie group (the bin's count plus the individuals
// equal to the value), individuals below it; a boundary or draw inside the
// group follows by arithmetic on the equal masses, and one pass over the
// registers counts the group's members in id order to name the id.  What
// fits none of this falls back to a bisection over selection keys that
// re-reads the row.
//
// Sources: "Transmuter.Generation (transmuter v2.0.0)", module doc (the
// processors and warpers, in order; temperature, top_k and top_p are the
// sampling warpers) and the inverse-CDF draw of a caller uniform over the
// kept ids in (score desc, id asc) order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "k_res_common.hpp"
#include "k_vkey.hpp"

namespace tsel {
namespace {

using namespace res;

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The map from key to bin: bin = min(max(k - bk1, 0), top), bk1 = first
// binned key - 1 (lower keys land in bin 0, which counts for nothing; keys
// past the last bin pile up there).  zn, zp: the bins of the two near-zero
// keys, or -1.
struct VMap {
  uint32_t bk1, top;
  int zn, zp;
};

__device__ __forceinline__ int vbin(uint32_t k, const VMap &m) {
  return min(max((int)k - (int)m.bk1, 0), (int)m.top);
}
// Key of bin b >= 1.
__device__ __forceinline__ uint32_t vbin_key(int b, const VMap &m) { return (uint32_t)b + m.bk1; }

// Packed form for the two bf16 scores of one word: the LDS byte addresses of
// their bins in this lane's histogram copy (lb: the copy's address in both
// halves; bins * 4 + lb stays below 2^16).  Constants sit in scalar
// registers (a literal cannot be an operand of the three-operand forms).
struct VMapP {
  u16x2 bk1, top;
  uint32_t lb, c7fff, czm, c8000;
};
__device__ __forceinline__ u16x2 vmag2(uint32_t w, const VMapP &m) {  // the clamped magnitudes
  return __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, w) & __builtin_bit_cast(u16x2, m.c7fff),
                                       __builtin_bit_cast(u16x2, m.czm));
}
__device__ __forceinline__ u16x2 vkeys2(uint32_t w, u16x2 t, const VMapP &m) {
  const u16x2 u = __builtin_bit_cast(u16x2, w);
  const i16x2 sx = __builtin_bit_cast(i16x2, u) >> (i16x2)(int16_t)15;
  uint32_t k;  // t ^ sx ^ 0x8000 in one three-input operation
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96"
      : "=v"(k)
      : "v"(__builtin_bit_cast(uint32_t, t)), "v"(__builtin_bit_cast(uint32_t, sx)), "s"(m.c8000));
  return __builtin_bit_cast(u16x2, k);
}
__device__ __forceinline__ u16x2 vkeys2(uint32_t w, const VMapP &m) {
  return vkeys2(w, vmag2(w, m), m);
}
__device__ __forceinline__ uint32_t vaddr2(uint32_t w, u16x2 t, const VMapP &m) {
  const u16x2 idx =
      __builtin_elementwise_min(__builtin_elementwise_sub_sat(vkeys2(w, t, m), m.bk1), m.top);
  uint32_t a;
  asm("v_pk_mad_u16 %0, %1, 4, %2 op_sel_hi:[1,0,1]"
      : "=v"(a)
      : "v"(__builtin_bit_cast(uint32_t, idx)), "v"(m.lb));
  return a;
}

// A constant in a scalar register (a literal cannot be an operand of the
// three-operand bit operations).
__device__ __forceinline__ uint32_t sconst(uint32_t v) {
  uint32_t r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}

// LDS address of a pointer into the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void lds_add(uint32_t addr, uint32_t v) {
  __hip_atomic_fetch_add((__attribute__((address_space(3))) uint32_t *)(uintptr_t)addr, v,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

constexpr int kTieCap = 128;
// A listed individual's id (below 2^18 on this path) carries its bin in the
// bits above, set when its score is known.
constexpr int kIdBits = 18;
constexpr int32_t kIdMask = (1 << kIdBits) - 1;
// A bin's count holds its dense elements in the low bits and, from the fixed
// point masses on, its listed individuals above them.
constexpr int kIndShift = 18;
constexpr uint32_t kDenseMask = (1u << kIndShift) - 1u;

struct VShared {
  BinView view, view2;  // (view2: the draw's bin when it is known before the boundary's walk)
  WalkResult walk[2];
  float gv[2];
  int gk[2];
  int gi[2], gw[2], gr[2];
  int gid[2];
  int wtot[16];
  int n_ind_b, n_tie_b, n_above_b;
  int n_ind_b2, n_tie_b2, n_above_b2;
  double mbp, mbq, sbase2;
  int tie_id[kTieCap];  // ids of the viewed bin's individuals equal to its value
  int tie_id2[kTieCap];
  int nz;
  uint32_t kmax[NW];
  float fmax[NW];
  int ovf;
  int view_ntie;  // the view's individuals equal to its value
};

template <int NT_>
__device__ __forceinline__ uint32_t block_max_u32_lds(uint32_t v, uint32_t *scratch) {
  constexpr int NW_ = NT_ / kWave;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  v = wave_max_u32_uni(v);  // (row moves, no LDS round trips)
  if (lane == 0) scratch[wid] = v;
  lds_barrier();
  return wave_max_u32_uni(lane < NW_ ? scratch[lane] : 0u);
}

// The map for a first binned key bk (>= the smallest finite key).
__device__ __forceinline__ VMap make_vmap(uint32_t bk) {
  VMap m;
  m.bk1 = bk - 1u;
  m.top = (uint32_t)(kVBins - 1);
  const int zn = vbin(kKeyZoneNeg, m), zp = vbin(kKeyZonePos, m);
  m.zn = zn >= 1 && zn < kVBins - 1 ? zn : -1;
  m.zp = zp >= 1 && zp < kVBins - 1 ? zp : -1;
  return m;
}
__device__ __forceinline__ VMapP pack_vmap(const VMap &m, uint32_t lb) {
  VMapP p;
  p.bk1 = (u16x2)(uint16_t)m.bk1;
  p.top = (u16x2)(uint16_t)m.top;
  p.lb = lb | (lb << 16);
  p.c7fff = sconst(0x7FFF7FFFu);
  p.czm = sconst(kZoneMag | (kZoneMag << 16));
  p.c8000 = sconst(0x80008000u);
  return p;
}

// First binned key for a maximum of key kmax: kDropNats below it.
__device__ __forceinline__ uint32_t base_key(uint32_t kmax) {
  if (kmax < kKeyLowFinite) return kKeyLowFinite;  // no finite score: from the lowest
  if (kmax == kKeyZoneNeg || kmax == kKeyZonePos) kmax = kKeyZonePos + 1u;  // (an upper bound)
  return max(vkey_floor(vkey_value(kmax) - kDropNats), kKeyLowFinite);
}

}  // namespace

static_assert(sizeof(RowShared) <= kVRowSharedBytes, "row scalars");
static_assert(sizeof(VShared) + kVRowSharedBytes <= kVSharedBytes, "kernel scalars");

template <int R>
__global__ __launch_bounds__(NT, 1) void k_vres(SelectArgs a) {
  using E = Elem<1>;
  constexpr int EPC = E::EPC;
  constexpr int PIPE0 = R < 4 ? R : 4;  // chunks asked for before the staging
  constexpr int PIPE = R < 4 ? R : 4;  // chunks in flight while counting
  constexpr int NB = kVBins;
  constexpr int BPT = (NB + NT - 1) / NT;
  // (no static LDS: the dynamic block starts at address 0, so histogram
  // offsets are LDS addresses as they stand)
  extern __shared__ __align__(16) unsigned char smem[];
  RowShared &sh = *reinterpret_cast<RowShared *>(smem + a.off_sh);
  VShared &vs = *reinterpret_cast<VShared *>(smem + a.off_sh + kVRowSharedBytes);
  const Lds s = carve(a, smem);
  uint16_t *woff = reinterpret_cast<uint16_t *>(smem + a.off_woff);
  const int tid = threadIdx.x, row = blockIdx.x, V = a.V;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const int NG = V / EPC;  // whole chunks (>= 1 on this path)
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  // ---- 0. the small loads: lengths, history, masks, tail --------------------
  // (the lengths are asked for first and read only after the clearing
  // below, so that their latency hides behind it; the loads issued in
  // between do not depend on them)
  RowInfo ri;
  const int len0 = __builtin_nontemporal_load(a.lens + row);
  const int len1 = __builtin_nontemporal_load(a.lens + a.B + row);
  const int len2 = __builtin_nontemporal_load(a.lens + 2 * a.B + row);
  const float u_row = __builtin_nontemporal_load(a.uniforms + row);  // (read at the draw)
  Early ea;
  early_loads<1>(a, row, rowp, ea);
  const int tail_n = V - NG * EPC;

  // ---- 1. staging: masks and list (LDS only) --------------------------------
  // LDS from byte 0: four histogram copies (u32 counts, kVStride words
  // apart); after the fold, copy 0 keeps the counts and the space of the
  // others holds the per-bin masses and the ordered view of one bin.
  uint32_t *cnt = reinterpret_cast<uint32_t *>(smem);
  double *bmass = reinterpret_cast<double *>(smem + kVMassOff);
  uint64_t *lfix = reinterpret_cast<uint64_t *>(smem + kVMassOff);
  uint64_t *okey = reinterpret_cast<uint64_t *>(smem + kVViewOff);
  float *oval = reinterpret_cast<float *>(okey + kGatherCap);
  uint64_t *gkey = reinterpret_cast<uint64_t *>(oval + kGatherCap);
  float *gval = reinterpret_cast<float *>(gkey + kGatherCap);
  // The row through a buffer resource (one offset register per lane, the
  // chunk's offset in a scalar; chunks past the row read as 0): its first
  // chunks are asked for now, before the clearing below, the others as the
  // chunks are counted.
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(rowp), (short)0, NG * 16, 0x00020000);
  auto load_chunk = [&](int i) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, tid * 16, i * NT * 16, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  };
  uint4 reg[R];
#pragma unroll
  for (int i = 0; i < PIPE0; ++i) reg[i] = load_chunk(i);
  // While the small loads fly: clear the histogram and the masks.  Both
  // masks run on to byte R * NT (one byte per chunk slot of the registers),
  // the kill mask with every slot past the row's ids marked removed, so that
  // chunk i's bytes sit at fixed offsets.
  {
    uint4 *c4 = reinterpret_cast<uint4 *>(cnt);
    for (int b = tid; b < kVCopies * kVStride / 4; b += NT) c4[b] = make_uint4(0u, 0u, 0u, 0u);
  }
  stage_clear(s, sh, R * NT / 4, (V + EPC - 1) / EPC, R * NT / 4);
  ri.L = __builtin_amdgcn_readfirstlane(len0);
  ri.P = __builtin_amdgcn_readfirstlane(len1);
  ri.M = __builtin_amdgcn_readfirstlane(len2);
  if (row_prologue_after_lens(a, row, ri)) return;
  if (lds_addr(smem) + kVHistBytes > 65536) {  // (not with this block's layout)
    if (tid == 0) a.out_tokens[row] = kPending;
    return;
  }
  const int32_t *h = a.hist + (int64_t)row * a.hist_stride;
  const int n_list = uni(stage(a, row, ri, s, sh, h, ea, woff));
  if (n_list < 0) return;

  // The seen ids' scores are gathered chunk index by chunk index, each right
  // after its chunk was asked for, so that they read the lines that chunk
  // brings in.  lbv[i]: the first list slot of chunk index i (the list is in
  // id order; chunk index i holds ids [i * NT * EPC, (i + 1) * NT * EPC)).
  // (lane i reads entry i; the entries then come out of the lanes)
  int lbv[R + 1];
  {
    const int w = lane * (NT * EPC / 32);
    const int lv = lane <= R ? (w < a.mw ? (int)woff[w] : n_list) : 0;
#pragma unroll
    for (int i = 0; i <= R; ++i) lbv[i] = __builtin_amdgcn_readlane(lv, i);
  }
  bool list_ovf = false;
#pragma unroll
  for (int i = 0; i < R; ++i) list_ovf |= lbv[i + 1] - lbv[i] > NT;
  const __amdgpu_buffer_rsrc_t rsg =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(rowp), (short)0, V * 2, 0x00020000);
  // (a lane past the chunk index's entries asks for an id far past the row:
  // its load reads nothing and returns 0, which no one uses)
  // (the list slot this thread takes for chunk index i: successive chunk
  // indices start a quarter of the workgroup further on, so that the
  // penalties of the gathered scores spread over every wave)
  auto slot_of = [&](int i) { return lbv[i] + ((tid + NT - (NT / 4) * (i & 3)) & (NT - 1)); };
  auto gather_id = [&](int i) {  // the id at list slot slot_of(i)
    const int k = slot_of(i);
    return k < lbv[i + 1] ? s.list_id[k] : 0x3FFFFFFF;
  };
  auto gather_at = [&](int id) -> uint32_t {
    return __builtin_amdgcn_raw_buffer_load_b16(rsg, id * 2, 0, 0);
  };
  auto gather = [&](int i) { return gather_at(gather_id(i)); };
  VMap vm;  // the value bins (placed by the first chunks, before any consume)
  // (a gathered score is penalized as it lands, and its bin noted beside its
  // id; lmax: the seen ids' top)
  float lmax = -INFINITY;
  auto consume = [&](int i, uint32_t raw) {
    const int k = slot_of(i);
    if (k < lbv[i + 1]) {
      const float y = penalize(__uint_as_float(raw << 16), a.rep);
      s.list_val[k] = y;
      s.list_id[k] |= vbin(vkey_floor(y), vm) << kIdBits;
      lmax = fmaxf(lmax, y);
    }
  };
  // (the bisection and the final scores read plain ids)
  auto untag = [&](int n) {
    __syncthreads();
    for (int k = tid; k < n; k += NT) s.list_id[k] &= kIdMask;
    __syncthreads();
  };
  uint32_t gr[R];
#pragma unroll
  for (int i = 0; i < PIPE0; ++i) gr[i] = gather(i);
#pragma unroll
  for (int i = PIPE0; i < PIPE; ++i) {
    reg[i] = load_chunk(i);
    gr[i] = gather(i);
  }

  // ---- 2. chunks as they land: count -----------------------------------------
  // this lane's histogram copy, as an LDS address (the block has no static
  // LDS, so the copies lie below 2^16 and bin addresses fit 16 bits)
  const uint32_t lb = lds_addr(cnt) + (uint32_t)(lane & (kVCopies - 1)) * kVStride * 4u;
  const uint32_t ninf = sconst(0xFF80FF80u);
  VMapP vp;
  // A near-zero score has a clamped magnitude of 0: every lane keeps the
  // least of its halves (the magnitudes stay below the binary16 infinity,
  // so a binary16 minimum orders them as integers), which tells the lanes
  // that hold one.
  uint32_t zacc = 0x7BFF7BFFu;
  auto count_chunk = [&](uint4 c) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    u16x2 t[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) t[q] = vmag2(w[q], vp);
    asm("v_pk_minimum3_f16 %0, %0, %1, %2"
        : "+v"(zacc)
        : "v"(__builtin_bit_cast(uint32_t, t[0])), "v"(__builtin_bit_cast(uint32_t, t[1])));
    asm("v_pk_minimum3_f16 %0, %0, %1, %2"
        : "+v"(zacc)
        : "v"(__builtin_bit_cast(uint32_t, t[2])), "v"(__builtin_bit_cast(uint32_t, t[3])));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a2 = vaddr2(w[q], t[q], vp);
      lds_add(a2 & 0xFFFFu, 1u);
      lds_add(a2 >> 16, 1u);
    }
  };
  // chunk i of this lane is chunk g = tid + i * NT: its kill byte is byte g
  // of the kill mask (read one chunk ahead, so that the read does not queue
  // behind the chunk's own histogram adds, and so are the list ids gathered)
  const uint8_t *kbyte = reinterpret_cast<const uint8_t *>(s.kmask) + tid;
  const int itail = tail_n > 0 ? NG / NT : -1, ttail = NG % NT;
  // (every lane loaded the same tail: it is held in scalar registers)
  tail_words<1>(ea, V);
  const uint32_t tw0 = uni(ea.tw[0]), tw1 = uni(ea.tw[1]), tw2 = uni(ea.tw[2]), tw3 = uni(ea.tw[3]);
  auto chunk_of = [&](int i) {  // (the tail, at its slot)
    uint4 c = launder(reg[i]);
    if (i == itail) {  // (uniform)
      const bool t = tid == ttail;
      c = make_uint4(t ? tw0 : c.x, t ? tw1 : c.y, t ? tw2 : c.z, t ? tw3 : c.w);
    }
    return c;
  };
  uint32_t kb_n = kbyte[0];
  int gid_n = PIPE < R ? gather_id(PIPE) : 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i + PIPE < R) {
      reg[i + PIPE] = load_chunk(i + PIPE);
      gr[i + PIPE] = gather_at(gid_n);
      if (i + PIPE + 1 < R) gid_n = gather_id(i + PIPE + 1);
    }
    const uint32_t kb = kb_n;
    if (i + 1 < R) kb_n = kbyte[(i + 1) * NT];
    const uint4 c = vkill(chunk_of(i), kb, ninf);
    reg[i] = c;
    if (i >= 1) consume(i - 1, gr[i - 1]);  // (asked for before chunk i)
    if (i == 0) {
      // the maximum of every lane's first chunk places the bins
      vp.c7fff = sconst(0x7FFF7FFFu);
      vp.czm = sconst(kZoneMag | (kZoneMag << 16));
      vp.c8000 = sconst(0x80008000u);
      u16x2 m2 = vkeys2(c.x, vp);
      m2 = __builtin_elementwise_max(m2, vkeys2(c.y, vp));
      m2 = __builtin_elementwise_max(m2, vkeys2(c.z, vp));
      m2 = __builtin_elementwise_max(m2, vkeys2(c.w, vp));
      const uint32_t km = max((uint32_t)m2.x, (uint32_t)m2.y);
      vm = make_vmap(base_key(uni(block_max_u32_lds<NT>(km, vs.kmax))));
      vp = pack_vmap(vm, lb);
    }
    count_chunk(c);
  }
  consume(R - 1, gr[R - 1]);
  if (list_ovf) {  // (uniform, rare) list slots past NT in one chunk index
    for (int e = tid; e < n_list; e += NT) {
      const int id = s.list_id[e] & kIdMask;
      if (e - (int)woff[id / (NT * EPC) * (NT * EPC / 32)] >= NT) {
        const float y = penalize(E::load1(rowp, id), a.rep);
        s.list_val[e] = y;
        s.list_id[e] = id | (vbin(vkey_floor(y), vm) << kIdBits);
        lmax = fmaxf(lmax, y);
      }
    }
  }
  __syncthreads();  // the row has landed
  // fold the copies (each thread its own bins, so no barrier between the
  // reads and the writes); the highest occupied bin and the seen ids' top
  // score in one workgroup reduction
  // (a thread's four bins are adjacent words: one 16-byte read per copy)
  static_assert(BPT == 4 && NB % 4 == 0 && kVStride % 4 == 0, "four bins a thread, 16-byte rows");
  uint32_t top_b = 0u;
  if (tid * BPT < NB) {
    uint4 c = reinterpret_cast<const uint4 *>(cnt)[tid];
#pragma unroll
    for (int k = 1; k < kVCopies; ++k) {
      const uint4 d = reinterpret_cast<const uint4 *>(cnt + k * kVStride)[tid];
      c.x += d.x;
      c.y += d.y;
      c.z += d.z;
      c.w += d.w;
    }
    reinterpret_cast<uint4 *>(cnt)[tid] = c;
    const int b0 = tid * BPT;
    if (c.x && b0 >= 1) top_b = (uint32_t)b0;
    if (c.y) top_b = (uint32_t)(b0 + 1);
    if (c.z) top_b = (uint32_t)(b0 + 2);
    if (c.w) top_b = (uint32_t)(b0 + 3);
  }
  {
    const uint32_t tw = wave_max_u32_uni(top_b);
    const float lw = wave_max_f32_uni(lmax);
    if (lane == 0) {
      vs.kmax[wid] = tw;
      vs.fmax[wid] = lw;
    }
    lds_barrier();
    top_b = lane < NW ? vs.kmax[lane] : 0u;
    lmax = lane < NW ? vs.fmax[lane] : -INFINITY;
  }
  const int btop = (int)wave_max_u32_uni(top_b);
  lmax = wave_max_f32_uni(lmax);
  const int zn = vm.zn, zp = vm.zp;  // the near-zero bins (or -1)
  // Scores past the last bin (the row's maximum far above its first
  // chunks'): the bisection decides.
  bool fallback = btop == NB - 1 || (lmax > -INFINITY && vbin(vkey_floor(lmax), vm) == NB - 1);
  if (tid == 0) {
    sh.n_list = n_list;
    sh.dense_pen = 0;
  }
  // the reference: an upper bound of the row's maximum (a near-zero bin:
  // its upper edge)
  const float kZone = __uint_as_float((uint32_t)(127 - kZoneExp) << 23);
  const float dmax = btop < 1 ? -INFINITY
                     : btop == zp ? kZone
                     : btop == zn ? 0.0f
                                  : vkey_value(vbin_key(btop, vm));
  const float mx = fmaxf(dmax, lmax);
  uint64_t kcut = 0ull;
  int token = 0;
  if (mx == -INFINITY) {  // every id removed: id 0, nothing kept
    if (tid == 0) {
      a.out_tokens[row] = 0;
      if (a.out_logprobs) a.out_logprobs[row] = lp_none();
    }
    if (a.out_processed) {
      untag(n_list);
      res_processed<1>(a, row, s, INFINITY, ~0ull, n_list);
    }
    return;
  }
  const float cref = mx * kLog2e;
  auto mass = [&](float y) { return __builtin_amdgcn_exp2f(fmaf(y, kLog2e, -cref)); };

  // ---- 3. near-zero members, individual masses, bin masses ---------------------
  // Near-zero members one by one, after the seen ids: (id, score), the two
  // near-zero bins then holding individuals only.  If there are too many
  // and they all hold one value (zeros, say), that value is a tie group in
  // its bin instead.
  int n_ind = n_list;
  float zval = -INFINITY;  // the value of that tie group
  int zgb = -1;            // its bin
  if ((zn >= 1 && cnt[zn] > 0u) || (zp >= 1 && cnt[zp] > 0u)) {
    if (tid == 0) vs.nz = 0;
    __syncthreads();
    float zlo = INFINITY, zhi = -INFINITY;
    // Lanes that saw one: which of their chunks hold one (a magnitude within
    // reach: max(|u| - Z, 0) is 0 in some half), one bit each; then those
    // chunks one at a time, picked from the registers by index.  (Short
    // code: it runs cold, on few rows and few waves.)
    if ((zacc & 0xFFFFu) == 0u || (zacc >> 16) == 0u) {
      const u16x2 zm = __builtin_bit_cast(u16x2, kZoneMag | (kZoneMag << 16));
      const u16x2 msk = __builtin_bit_cast(u16x2, 0x7FFF7FFFu);
      auto near = [&](uint32_t w) {  // per half: 0 where the magnitude is in reach
        return __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, w) & msk, zm);
      };
      uint32_t zb = 0u;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const uint4 c = reg[i];
        u16x2 t = __builtin_elementwise_min(near(c.x), near(c.y));
        t = __builtin_elementwise_min(t, __builtin_elementwise_min(near(c.z), near(c.w)));
        zb |= (t.x == 0 || t.y == 0) ? 1u << i : 0u;
      }
      while (zb) {
        const int i = __ffs(zb) - 1;
        zb &= zb - 1u;
        uint4 c = reg[0];
#pragma unroll
        for (int k = 1; k < R; ++k)
          if (i == k) c = reg[k];
        const int g = tid + i * NT;
        for (int j = 0; j < EPC; ++j) {
          const float x = E::get(c, j);
          if (fabsf(x) <= kZone) {
            zlo = fminf(zlo, x);
            zhi = fmaxf(zhi, x);
            const int slot = atomicAdd(&vs.nz, 1);
            if (slot < kZoneCap) {
              s.list_id[n_list + slot] = (g * EPC + j) | (vbin(vkey_floor(x), vm) << kIdBits);
              s.list_val[n_list + slot] = x;
            }
          }
        }
      }
    }
    __syncthreads();
    const int nz = uni(vs.nz);
    if (nz > kZoneCap) {  // too many to list: are they all one value?
      zlo = -uni(block_max_f32<NT>(-zlo, sh.red_f32));
      zhi = uni(block_max_f32<NT>(zhi, sh.red_f32));
    }
    if (nz <= kZoneCap) {
      n_ind = n_list + nz;
      if (tid == 0) {  // the members are individuals now
        if (zn >= 1) cnt[zn] = 0u;
        if (zp >= 1) cnt[zp] = 0u;
      }
    } else if (zlo == zhi) {
      zval = zlo + 0.0f;  // (-0 is +0; zeros of both signs join in the upper bin)
      zgb = zval >= 0.0f ? zp : zn;
      if (zgb < 1) {
        fallback = true;
      } else if (zval == 0.0f && zn >= 1 && tid == 0) {
        cnt[zp] += cnt[zn];
        cnt[zn] = 0u;
      }
    } else {
      fallback = true;
    }
  }
  // Value of bin b (-inf for a near-zero bin of individuals only) and its
  // fixed-point unit: the ulp of the mass of the bin's lowest score, which
  // every individual of the bin reaches or exceeds.
  auto bin_value = [&](int b) {
    return b == zgb ? zval : (b == zn || b == zp) ? -INFINITY : vkey_value(vbin_key(b, vm));
  };
  auto unit_expo = [&](int b) {
    const float lo = b == zn ? -kZone : b == zp ? 0.0f : vkey_value(vbin_key(b, vm));
    return (int)((__float_as_uint(mass(lo)) >> 23) & 0xFFu);
  };
  for (int b = tid; b < NB; b += NT) lfix[b] = 0ull;
  if (tid == 0) vs.ovf = 0;
  __syncthreads();
  // (a thread takes four adjacent entries, read in one 16-byte access per
  // array; their adds are independent of each other)
  static_assert(kGatherCap % 4 == 0, "16-byte list rows");
  for (int k0 = 4 * tid; k0 < n_ind; k0 += 4 * NT) {
    const int4 i4 = *reinterpret_cast<const int4 *>(s.list_id + k0);
    const float4 y4 = *reinterpret_cast<const float4 *>(s.list_val + k0);
    const int iq[4] = {i4.x, i4.y, i4.z, i4.w};
    const float yq[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = iq[q] >> kIdBits;
      if (k0 + q >= n_ind || b < 1) continue;
      atomicAdd(&cnt[b], 1u << kIndShift);
      const int eu = unit_expo(b);
      const uint32_t eb = __float_as_uint(mass(yq[q]));
      const int ek = (int)((eb >> 23) & 0xFFu);
      if (eu == 0 || ek == 0) continue;  // below 2^-126 of the maximum: nothing
      const int sft = ek - eu;
      if (sft < 0 || sft > 24) { vs.ovf = 1; continue; }
      atomicAdd(reinterpret_cast<unsigned long long *>(&lfix[b]),
                (unsigned long long)((eb & 0x7FFFFFu) | 0x800000u) << sft);
    }
  }
  __syncthreads();
  if (uni(vs.ovf) != 0) fallback = true;
  // bin masses, in place of the fixed-point sums
  // (a thread's four bins come in 16-byte reads and leave in 16-byte writes)
  double part = 0.0;
  if (tid * BPT < NB) {
    const uint4 n4 = reinterpret_cast<const uint4 *>(cnt)[tid];
    const ulonglong2 la = reinterpret_cast<const ulonglong2 *>(lfix)[2 * tid];
    const ulonglong2 lb = reinterpret_cast<const ulonglong2 *>(lfix)[2 * tid + 1];
    const uint32_t nq[4] = {n4.x, n4.y, n4.z, n4.w};
    const uint64_t lq[4] = {la.x, la.y, lb.x, lb.y};
    double mq[4];
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      const int b = tid * BPT + q;
      double m = 0.0;
      if (b >= 1) {
        const uint32_t n = nq[q] & kDenseMask;
        if (n) m = (double)n * (double)mass(bin_value(b));
        if (lq[q]) {
          const int eu = unit_expo(b);
          m += (double)lq[q] * __longlong_as_double((long long)(eu - 150 + 1023) << 52);
        }
      }
      mq[q] = m;
      part += m;
    }
    reinterpret_cast<double2 *>(bmass)[2 * tid] = make_double2(mq[0], mq[1]);
    reinterpret_cast<double2 *>(bmass)[2 * tid + 1] = make_double2(mq[2], mq[3]);
  }

  // ---- 4. cumulative masses: the boundary bin and the draw bin -------------
  // Thread t owns bins [t*BPT, t*BPT + BPT); C(b) = mass of bins >= b.
  double incl;  // mass of bins owned by threads >= tid
  double W;     // the row's mass (every thread sums the wave totals alike)
  {
    const double v = wave_suffix_scan_f64_dpp(part);
    if (lane == 0) sh.red_f64[wid] = v;
    if (tid == 0) {
      sh.bin_p = -1;
      sh.bin_hi = -1;  // (the draw's bin, searched after the boundary's walk)
      vs.n_ind_b = 0;  // (the counters of the first view)
      vs.n_tie_b = 0;
      vs.n_above_b = 0;
      vs.n_ind_b2 = 0;  // (and of the predicted draw's view)
      vs.n_tie_b2 = 0;
      vs.n_above_b2 = 0;
    }
    __syncthreads();
    double after = 0.0;
    W = 0.0;
#pragma unroll
    for (int q = NW - 1; q >= 0; --q) {
      const double t = sh.red_f64[q];
      if (q > wid) after += t;
      W += t;
    }
    incl = v + after;
    W = uni(W);
  }
  // (the mass above this thread's bins waits in LDS: registers are scarce
  // while the row is held)
  double *above = reinterpret_cast<double *>(smem + kVAboveOff);
  above[tid] = incl - part;
  const bool use_top_p = a.top_p < 1.0f;
  const double pw = (double)a.top_p * W;
  const double u = (double)uni(u_row);
  if (tid * BPT < NB) {
    double C = above[tid];
    const double2 ma = reinterpret_cast<const double2 *>(bmass)[2 * tid];
    const double2 mb = reinterpret_cast<const double2 *>(bmass)[2 * tid + 1];
    const double mq[4] = {ma.x, ma.y, mb.x, mb.y};
#pragma unroll
    for (int q = BPT - 1; q >= 0; --q) {
      const int b = tid * BPT + q;
      const double Cb1 = C;
      C += mq[q];
      if (use_top_p && Cb1 < pw && C >= pw) {
        sh.bin_p = b;
        sh.sbase = Cb1;
        vs.mbp = mq[q];
      }
    }
  }
  __syncthreads();
  const int bp = uni(sh.bin_p);
  const double C_bp1 = bp >= 0 ? uni(sh.sbase) : 0.0;  // mass above the boundary bin
  const double m_bp = bp >= 0 ? uni(vs.mbp) : 0.0;     // the boundary bin's own mass

  // View of bin b (all threads): its value, its individuals other than the
  // value ordered by key into okey / oval, the tie group's size.  Returns
  // false when the bin has more individuals than fit.
  // The counters start at zero (cleared before an earlier barrier); the
  // view is written by thread 0 and read by its own wave until the next
  // barrier.
  auto view_bin = [&](int b) -> bool {
    const float v = bin_value(b);
    const uint32_t cb_ = uni(cnt[b]);
    if ((cb_ >> kIndShift) == 0u) {  // (no individuals: the view is the group alone)
      if (tid == 0) {
        vs.view.single = 1;
        vs.view.v = v;
        vs.view.e = v == -INFINITY ? 0.0f : mass(v);
        vs.view.n_ind = 0;
        vs.view.n_above = 0;
        vs.view.n_group = (int)(cb_ & kDenseMask);
        vs.view_ntie = 0;
      }
      return true;
    }
    for (int k = tid; k < n_ind; k += NT) {
      const int tagged = s.list_id[k];
      if ((tagged >> kIdBits) != b) continue;
      const float y = s.list_val[k];
      const int id = tagged & kIdMask;
      if (y == v) {
        const int slot = atomicAdd(&vs.n_tie_b, 1);
        if (slot < kTieCap) vs.tie_id[slot] = id;
      } else {
        const int slot = atomicAdd(&vs.n_ind_b, 1);
        if (slot < kGatherCap) {
          gkey[slot] = sel_key(y, (uint32_t)id);
          gval[slot] = mass(y);
        }
      }
    }
    __syncthreads();
    const int ni = uni(vs.n_ind_b);
    if (ni > kGatherCap) return false;
    for (int i = tid; i < ni; i += NT) {
      const uint64_t ki = gkey[i];
      int r = 0;
      for (int j = 0; j < ni; ++j) r += gkey[j] > ki;
      okey[r] = ki;
      oval[r] = gval[i];
      if (key_score(ki) > v) atomicAdd(&vs.n_above_b, 1);
    }
    // (up to 64 individuals were ordered by wave 0 alone, which also writes
    // and walks the view: no barrier then, only an order among its lanes;
    // the other waves touch none of the view's arrays meanwhile)
    if (ni > kWave) __syncthreads();
    else __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (tid == 0) {
      const int na = vs.n_above_b;
      vs.view.single = 1;
      vs.view.v = v;
      vs.view.e = v == -INFINITY ? 0.0f : mass(v);
      vs.view.n_ind = ni;
      vs.view.n_above = na;
      vs.view.n_group = (int)(cnt[b] & kDenseMask) + vs.n_tie_b;
      vs.view_ntie = vs.n_tie_b;
    }
    return true;
  };

  // (the walks run on wave 0 alone; the others wait at the barrier after)
  double Wp = W;
  int cut_kind = kNone, draw_kind = kNone;
  int cut_pos = 0x7FFFFFFF;
  int cut_rank = -1;  // kGroup cut: the boundary group's members kept, less one
  int bs = -1;
  double bs_start = 0.0;
  // The count pass for the draw's member (all threads), run while wave 0
  // walks the draw's bin: every lane counts the members of the bin's value
  // vv in each of its chunks (a nonzero value by its bf16 pattern, a zero
  // one by the pattern less the sign; seen ids equal to the value added from
  // the list), in byte fields, summed over rows of 16 lanes by shifts within
  // the row, into rsum.  Seen ids equal to vv are marked per thread and
  // chunk, 16 bits per thread, two threads a word, over the per-thread
  // masses above (idle once the draw's bin is found); rsum follows them
  // there, clear of the arrays the view's ordering reads.
  float vv = 0.0f;
  uint32_t pat = 0u, msk = 0xFFFFFFFFu, tmask = 0u;
  bool ltie_all = false;
  uint32_t *tiew = reinterpret_cast<uint32_t *>(above);
  uint32_t *rsum = tiew + NT / 2;  // 64 rows x 16 bytes
  static_assert(4 * (NT / 2) + 64 * 16 <= 8 * NT, "tie words and row sums within the masses");
  auto list_ties = [&](int i) {  // seen ids of chunk i equal to vv, per element bit j
    uint32_t mb = 0u;
    if ((tmask >> i) & 1u) {
      const int g = tid + i * NT;
      uint32_t bits = chunk_bits<1>(s.smask, g);
      while (bits) {
        const int j = __ffs(bits) - 1;
        bits &= bits - 1;
        if (s.list_val[list_slot(g * EPC + j, s.smask, woff)] == vv) mb |= 1u << j;
      }
    }
    return mb;
  };
  auto count_setup = [&](float v, int ntie, const int *tie_ids) {  // (ntie: the view's individuals equal to v)
    vv = v;
    ltie_all = ntie > 0;
    if (ltie_all) {
      for (int q = tid; q < NT / 2; q += NT) tiew[q] = 0u;
      __syncthreads();
      auto mark = [&](int id) {
        const int gg = id / EPC, t = gg % NT, ci = gg / NT;
        atomicOr(&tiew[t >> 1], 1u << ((t & 1) * 16 + ci));
      };
      if (ntie <= kTieCap) {
        if (tid < ntie) mark(tie_ids[tid]);
      } else {
        for (int k = tid; k < n_list; k += NT)
          if (s.list_val[k] == vv) mark(s.list_id[k] & kIdMask);
      }
      __syncthreads();
      tmask = (tiew[tid >> 1] >> ((tid & 1) * 16)) & 0xFFFFu;
    }
    pat = vv == 0.0f ? 0u : (__float_as_uint(vv) >> 16) * 0x10001u;
    msk = vv == 0.0f ? 0x7FFF7FFFu : 0xFFFFFFFFu;
  };
  auto count_rows = [&]() {
    // (a member leaves a zero half in (w & msk) ^ pat; 1 - that half,
    // saturated, is 1 exactly there; the four words' halves are added in
    // place and the two halves by a dot product with (1, 1))
    const u16x2 one2 = {1, 1};
    auto members = [&](const uint4 &c) -> uint32_t {
      const uint32_t w[4] = {c.x, c.y, c.z, c.w};
      u16x2 y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        y[q] = __builtin_elementwise_sub_sat(one2, __builtin_bit_cast(u16x2, (w[q] & msk) ^ pat));
      return __builtin_amdgcn_udot2((y[0] + y[1]) + (y[2] + y[3]), one2, 0u, false);
    };
    uint32_t cb[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < R; ++i) {
      cb[i >> 2] |= members(reg[i]) << ((i & 3) * 8);
      __builtin_amdgcn_sched_barrier(0);  // one chunk at a time: the row holds the registers
    }
    if (ltie_all) {
#pragma unroll
      for (int i = 0; i < R; ++i) cb[i >> 2] += (uint32_t)__popc(list_ties(i)) << ((i & 3) * 8);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // inclusive sums along each row of 16 lanes
      cb[k] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cb[k], 0x111, 0xF, 0xF, true);
      cb[k] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cb[k], 0x112, 0xF, 0xF, true);
      cb[k] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cb[k], 0x114, 0xF, 0xF, true);
      cb[k] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cb[k], 0x118, 0xF, 0xF, true);
    }
    // (rows numbered wave * 4 + row: that is id order within a chunk index)
    if ((lane & 15) == 15) {
      const int u = wid * 4 + (lane >> 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) rsum[u * 4 + k] = cb[k];
    }
  };

  // The draw's bin before the boundary's walk: the kept mass lies between
  // the mass above the boundary bin and that plus the bin's own, so the
  // draw's target lies between u times either.  When both ends fall inside
  // one bin above the boundary bin, that bin is the draw's: its view and
  // the count of its value's members then run beside the boundary's walk.
  uint64_t *okey2 = reinterpret_cast<uint64_t *>(smem + kVView2Off);
  float *oval2 = reinterpret_cast<float *>(okey2 + kGatherCap2);
  uint64_t *gkey2 = reinterpret_cast<uint64_t *>(oval2 + kGatherCap2);
  float *gval2 = reinterpret_cast<float *>(gkey2 + kGatherCap2);
  {
    const double tlo = u * (bp >= 0 ? C_bp1 : W), thi = u * (bp >= 0 ? C_bp1 + m_bp : W);
    if (!fallback && tid * BPT < NB) {
      double C = above[tid];
      const double2 ma = reinterpret_cast<const double2 *>(bmass)[2 * tid];
      const double2 mb = reinterpret_cast<const double2 *>(bmass)[2 * tid + 1];
      const double mq[4] = {ma.x, ma.y, mb.x, mb.y};
#pragma unroll
      for (int q = BPT - 1; q >= 0; --q) {
        const int b = tid * BPT + q;
        const double m = mq[q];
        if (b >= 1 && b > bp && m > 0.0 && C <= tlo && thi < C + m) {
          sh.bin_hi = b;
          vs.sbase2 = C;
          vs.mbq = m;
        }
        C += m;
      }
    }
  }
  __syncthreads();
  const int bq = fallback ? -1 : uni(sh.bin_hi);
  bool pred = false;
  if (bq >= 0) {
    // both views in one pass over the list
    const float v0 = bp >= 0 ? bin_value(bp) : 0.0f, v1 = bin_value(bq);
    const bool need0 = bp >= 0 && (uni(cnt[bp]) >> kIndShift) != 0u;
    const bool need1 = (uni(cnt[bq]) >> kIndShift) != 0u;
    if (need0 || need1) {
      for (int k = tid; k < n_ind; k += NT) {
        const int tagged = s.list_id[k];
        const int tb = tagged >> kIdBits;
        if (tb != bp && tb != bq) continue;
        const float y = s.list_val[k];
        const int id = tagged & kIdMask;
        const bool one = tb == bq;
        if (y == (one ? v1 : v0)) {
          const int slot = atomicAdd(one ? &vs.n_tie_b2 : &vs.n_tie_b, 1);
          if (slot < kTieCap) (one ? vs.tie_id2 : vs.tie_id)[slot] = id;
        } else {
          const int slot = atomicAdd(one ? &vs.n_ind_b2 : &vs.n_ind_b, 1);
          if (slot < (one ? kGatherCap2 : kGatherCap)) {
            (one ? gkey2 : gkey)[slot] = sel_key(y, (uint32_t)id);
            (one ? gval2 : gval)[slot] = mass(y);
          }
        }
      }
      __syncthreads();
    }
    const int n0 = need0 ? uni(vs.n_ind_b) : 0, n1 = need1 ? uni(vs.n_ind_b2) : 0;
    const int t0 = need0 ? uni(vs.n_tie_b) : 0, t1 = need1 ? uni(vs.n_tie_b2) : 0;
    // (each view ordered by one wave: at most 64 individuals each)
    pred = n0 <= kWave && n1 <= kGatherCap2 && t0 <= kTieCap && t1 <= kTieCap;
    if (!pred) {
      if (tid == 0) {  // (the counters start again for the views taken one by one)
        vs.n_ind_b = 0;
        vs.n_tie_b = 0;
        vs.n_above_b = 0;
      }
      __syncthreads();
    } else {
      if (wid == 0 && lane < n0) {
        const uint64_t ki = gkey[lane];
        int r = 0;
        for (int j = 0; j < n0; ++j) r += gkey[j] > ki;
        okey[r] = ki;
        oval[r] = gval[lane];
        if (key_score(ki) > v0) atomicAdd(&vs.n_above_b, 1);
      }
      if (wid == 1 && lane < n1) {
        const uint64_t ki = gkey2[lane];
        int r = 0;
        for (int j = 0; j < n1; ++j) r += gkey2[j] > ki;
        okey2[r] = ki;
        oval2[r] = gval2[lane];
        if (key_score(ki) > v1) atomicAdd(&vs.n_above_b2, 1);
      }
      __syncthreads();
      if (tid == 0) {
        if (bp >= 0) {
          vs.view.single = 1;
          vs.view.v = v0;
          vs.view.e = v0 == -INFINITY ? 0.0f : mass(v0);
          vs.view.n_ind = n0;
          vs.view.n_above = need0 ? vs.n_above_b : 0;
          vs.view.n_group = (int)(cnt[bp] & kDenseMask) + t0;
        }
        vs.view2.single = 1;
        vs.view2.v = v1;
        vs.view2.e = v1 == -INFINITY ? 0.0f : mass(v1);
        vs.view2.n_ind = n1;
        vs.view2.n_above = need1 ? vs.n_above_b2 : 0;
        vs.view2.n_group = (int)(cnt[bq] & kDenseMask) + t1;
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      count_setup(v1, t1, vs.tie_id2);
      const double sb2 = uni(vs.sbase2), mb2 = uni(vs.mbq);
      if (uni(wid) == 0) {
        // the boundary's walk gives the kept mass, hence the draw's target,
        // which must fall in the predicted bin
        double wp = W;
        if (bp >= 0) {
          wave_walk(true, C_bp1, pw, vs.view, okey, oval, 0x7FFFFFFF, &vs.walk[0]);
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
          wp = vs.walk[0].acc;
        }
        const double tg = u * wp;
        if (tg >= sb2 && tg < sb2 + mb2) {
          wave_walk(false, sb2, tg, vs.view2, okey2, oval2, 0x7FFFFFFF, &vs.walk[1]);
        } else if (lane == 0) {
          vs.walk[1].kind = kFail;  // (rounding put it elsewhere: the bisection)
        }
      }
      count_rows();  // (wave 0 after its walks, the others meanwhile)
      __syncthreads();
      if (bp >= 0) {
        cut_kind = uni(vs.walk[0].kind);
        if (cut_kind == kFail) fallback = true;
        Wp = uni(vs.walk[0].acc);
        cut_pos = uni(vs.walk[0].pos);
        cut_rank = uni(vs.walk[0].rank);
        if (cut_kind == kInd) kcut = uni(vs.walk[0].key);
      }
      bs = bq;
      bs_start = sb2;
      draw_kind = uni(vs.walk[1].kind);
      if (draw_kind == kFail) fallback = true;
    }
  }
  if (!pred) {
    if (!fallback && bp >= 0) {
      if (!view_bin(bp)) {
        fallback = true;
      } else {
        if (uni(wid) == 0) {
          wave_walk(true, C_bp1, pw, vs.view, okey, oval, 0x7FFFFFFF, &vs.walk[0]);
        }
        __syncthreads();
        cut_kind = uni(vs.walk[0].kind);
        if (cut_kind == kFail) fallback = true;
        Wp = uni(vs.walk[0].acc);
        cut_pos = uni(vs.walk[0].pos);
        cut_rank = uni(vs.walk[0].rank);
        if (cut_kind == kInd) kcut = uni(vs.walk[0].key);
      }
    }
    const double target = u * Wp;
    // The draw's bin: the bin whose cumulative mass interval holds the target
    // (bp counts only its kept part); every thread checks its own bins.
    if (!fallback) {
      // (the counters of a second view, first counted after the barrier that
      // ends the search)
      if (tid == 0) {
        vs.n_ind_b = 0;
        vs.n_tie_b = 0;
        vs.n_above_b = 0;
      }
      if (tid * BPT < NB) {
        double C = above[tid];
        const double2 ma = reinterpret_cast<const double2 *>(bmass)[2 * tid];
        const double2 mb = reinterpret_cast<const double2 *>(bmass)[2 * tid + 1];
        const double mq[4] = {ma.x, ma.y, mb.x, mb.y};
  #pragma unroll
        for (int q = BPT - 1; q >= 0; --q) {
          const int b = tid * BPT + q;
          if (b < 1) continue;
          const double m = (bp >= 0 && b == bp) ? (Wp - C_bp1) : mq[q];
          if (m > 0.0 && C <= target && target < C + m && (bp < 0 || b >= bp)) {
            sh.bin_hi = b;
            sh.sbase = C;
          }
          C += m;
        }
      }
      __syncthreads();
      bs = uni(sh.bin_hi);
      bs_start = uni(sh.sbase);
      if (bs < 0) {
        fallback = true;  // rounding left the target outside every bin
      } else {
        // (the same bin as the boundary: the view is still in place)
        const bool same = bs == bp && bp >= 0;
        if (!same && !view_bin(bs)) {
          fallback = true;
        } else {
          count_setup(bin_value(bs), same ? uni(vs.view_ntie) : uni(vs.n_tie_b), vs.tie_id);
          if (uni(wid) == 0) {
            wave_walk(false, bs_start, target, vs.view, okey, oval, same ? cut_pos : 0x7FFFFFFF, &vs.walk[1]);
          }
          count_rows();  // (wave 0 after its walk, the others meanwhile)
          __syncthreads();
          draw_kind = uni(vs.walk[1].kind);
        }
      }
      if (draw_kind == kFail) fallback = true;
    }
  }

  // ---- 5. one pass over the registers: the draw's rank in its tie group -----
  // (The boundary's own member is needed only for the final scores: such a
  // call takes the bisection when the boundary falls inside a tie group.)
  if (!fallback && a.out_processed && cut_kind == kGroup) fallback = true;
  const bool g1 = !fallback && draw_kind == kGroup;
  if (g1) {
    if (tid == 0) {
      vs.gk[1] = vs.walk[1].rank + 1;
      vs.gi[1] = -1;
      vs.gid[1] = -1;
    }
    // (the members were counted while the draw was walked)
    // wave wid scans chunk index wid over the 64 rows (lane = row)
    int rc = 0, rinc = 0;
    if (wid < R) {
      rc = (int)((rsum[lane * 4 + (wid >> 2)] >> ((wid & 3) * 8)) & 0xFFu);
      rinc = wave_incl_scan_i32(rc);
      if (lane == kWave - 1) vs.wtot[wid] = rinc;  // the chunk index's total
    }
    __syncthreads();
    // (inclusive sums within a row of 16 lanes by row moves)
    auto row16_incl_scan = [](int v) {
      v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
      v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
      v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
      v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
      return v;
    };
    if (wid == 0) {
      const int T = lane < R ? vs.wtot[lane] : 0;
      const int inc = row16_incl_scan(T);
      const int k = vs.gk[1];
      if (lane < 16 && inc - T < k && k <= inc) {
        vs.gi[1] = lane;
        vs.gr[1] = k - (inc - T);
      }
    }
    __syncthreads();
    const int ii = uni(vs.gi[1]);
    if (ii >= 0) {
      // every wave scans the rows of chunk index ii again and names the row
      // that holds the member; its wave goes on
      const int k = uni(vs.gr[1]);
      const int rc2 = (int)((rsum[lane * 4 + (ii >> 2)] >> ((ii & 3) * 8)) & 0xFFu);
      const int rinc2 = wave_incl_scan_i32(rc2);
      const uint64_t hit = __ballot(rinc2 - rc2 < k && k <= rinc2);
      const int ur = hit ? __ffsll((unsigned long long)hit) - 1 : -1;
      const int r0 = k - __builtin_amdgcn_readlane(rinc2 - rc2, ur < 0 ? 0 : ur);  // rank in its row
      if (ur >= 0 && wid == ur / 4 && (lane >> 4) == ur % 4) {
        // members among this lane's elements of chunk ii (the chunk picked
        // by a chain of selects: indexing reg[ii] at run time would send
        // the whole row through scratch memory)
        uint4 c = reg[0];
#pragma unroll
        for (int k = 1; k < R; ++k)
          if (ii == k) c = reg[k];
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
        uint32_t mbits = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = (w[q] & msk) ^ pat;
          mbits |= ((x & 0xFFFFu) == 0u ? 1u : 0u) << (2 * q);
          mbits |= ((x >> 16) == 0u ? 1u : 0u) << (2 * q + 1);
        }
        if (ltie_all) mbits |= list_ties(ii);
        const int cnt_l = __popc(mbits);
        const int inc = row16_incl_scan(cnt_l);
        if (inc - cnt_l < r0 && r0 <= inc) {
          int r = r0 - (inc - cnt_l);
          uint32_t bits = mbits;
          int j = 0;
          while (bits) {
            j = __ffs(bits) - 1;
            bits &= bits - 1;
            if (--r == 0) break;
          }
          vs.gid[1] = (tid + ii * NT) * EPC + j;
        }
      }
      __syncthreads();
    }
  }
  if (g1 && vs.gid[1] < 0) fallback = true;
  if (!fallback && draw_kind == kGroup) token = vs.gid[1];
  if (!fallback && draw_kind == kInd) token = (int)key_index(vs.walk[1].key);

  // ---- 6. the token's log-probability ("Log-probabilities") --------------
  // The log-softmax of the kept scores at the token, in binary64 from the
  // counts: every bin above the boundary's keeps its dense members (one
  // value: count * exp(v - mx)); the boundary bin keeps (cut_rank + 1)
  // members of its tie group, or, cut at an individual, its group when the
  // value lies above the cut; individuals are kept by bin and by key.  mx
  // bounds the row's scores from above (any shift gives the same value).
  // A row whose kept set reaches the dropped scores (no boundary, and some
  // scores below the bins), or that took the bisection, sums over the row
  // from memory instead.
  float lp = 0.0f;
  bool lp_row = fallback;
  if (a.out_logprobs && !fallback) {
    if (bp < 0 && (uni(cnt[0]) & kDenseMask) != 0u) {
      lp_row = true;
    } else {
      const double M = (double)mx;
      const float yt = draw_kind == kGroup ? bin_value(bs) : key_score(vs.walk[1].key);
      const float vcut = bp >= 0 ? bin_value(bp) : 0.0f;
      const float scut = cut_kind == kInd ? key_score(kcut) : 0.0f;
      double acc = 0.0;
      if (tid * BPT < NB) {
        const uint4 n4 = reinterpret_cast<const uint4 *>(cnt)[tid];
        const uint32_t nq[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
          const int b = tid * BPT + q;
          const uint32_t n = nq[q] & kDenseMask;
          if (b < 1 || n == 0u) continue;
          const float v = bin_value(b);
          if (!(v > -INFINITY)) continue;
          if (bp < 0 || b > bp || (b == bp && cut_kind == kInd && v > scut))
            acc += (double)n * exp((double)v - M);
        }
      }
      for (int k = tid; k < n_ind; k += NT) {
        const int tagged = s.list_id[k];
        const float y = s.list_val[k];
        if (!(y > -INFINITY)) continue;
        const int b = tagged >> kIdBits;
        const bool kept =
            bp < 0 || b > bp ||
            (b == bp && (cut_kind == kGroup ? y > vcut
                                            : sel_key(y, (uint32_t)(tagged & kIdMask)) >= kcut));
        if (kept) acc += exp((double)y - M);
      }
      if (tid == 0 && cut_kind == kGroup) acc += (double)(cut_rank + 1) * exp((double)vcut - M);
      const double Wk = block_sum_f64<NT>(acc, sh.red_f64);
      lp = (float)(((double)yt - M) - log(Wk));
    }
  }

  if (fallback || a.out_processed || lp_row) untag(n_ind);
  if (fallback) token = bisect_select<1, true>(a, row, s, sh, -INFINITY, cref, &kcut);
  if (a.out_logprobs && lp_row) lp = kept_logprob<1, true>(a, row, s, sh, -INFINITY, kcut, token);
  if (tid == 0) {
    a.out_tokens[row] = token;
    if (a.out_logprobs) a.out_logprobs[row] = lp;
  }
  if (a.out_processed) res_processed<1>(a, row, s, -INFINITY, kcut, n_list);
}

template <int R>
static hipError_t launch_vres_t(const SelectArgs &a, size_t lds, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};  // devices where the limit is raised
  const void *fn = reinterpret_cast<const void *>(&k_vres<R>);
  if (hipError_t e = ensure_dyn_lds(fn, (int)kVMaxDynLds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL((k_vres<R>), dim3(a.B), dim3(NT), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_vres(const SelectArgs &a, int res, size_t lds, hipStream_t st) {
  if (a.dtype != 1) return hipErrorInvalidValue;
  if (res == 16) return launch_vres_t<16>(a, lds, st);
  if (res == 8) return launch_vres_t<8>(a, lds, st);
  return launch_vres_t<4>(a, lds, st);
}

}  // namespace tsel
