// tsel_api.cpp -- the C ABI of libtsel.so (declared in include/tsel.h):
// argument validation on the host, on-chip layout of the selection kernel,
// and the launches.  No entry point prints, throws or exits.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "tsel.h"
#include "tsel_internal.hpp"

namespace {

constexpr int32_t kMaxVocab = 524288;   // on-chip kill + seen masks: V / 4 bytes
constexpr int32_t kMaxList = 8192 + 8;  // sparse list: distinct seen ids + row tail

inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

static_assert(TSEL_NOALLOC_SCRATCH_BYTES == tsel::kNoAllocScratchBytes, "one limit");

tsel_status check_params(const tsel_params *p, bool uniforms_given) {
  if (!p) return TSEL_ERR_INVALID_ARG;
  if (p->batch < 0 || p->vocab < 1) return TSEL_ERR_INVALID_ARG;
  if (p->logits_row_stride < p->vocab) return TSEL_ERR_INVALID_ARG;
  if (p->dtype != TSEL_F32 && p->dtype != TSEL_BF16) return TSEL_ERR_INVALID_ARG;
  if (p->hist_stride < 0) return TSEL_ERR_INVALID_ARG;
  if (!(p->repetition_penalty > 0.0f)) return TSEL_ERR_INVALID_ARG;
  if (p->no_repeat_ngram_size < 0) return TSEL_ERR_INVALID_ARG;
  if (p->min_length < 0 || p->min_new_tokens < 0) return TSEL_ERR_INVALID_ARG;
  if (p->n_eos < 0 || p->n_eos > TSEL_MAX_EOS) return TSEL_ERR_INVALID_ARG;
  if (p->do_sample) {
    if (!(p->temperature > 0.0f)) return TSEL_ERR_INVALID_ARG;
    if (p->top_k < 0) return TSEL_ERR_INVALID_ARG;
    if (!(p->top_p > 0.0f && p->top_p <= 1.0f)) return TSEL_ERR_INVALID_ARG;
    if (!uniforms_given) return TSEL_ERR_INVALID_ARG;
  }
  if (p->vocab > kMaxVocab) return TSEL_ERR_UNSUPPORTED;
  return TSEL_OK;
}

// On-chip layout of one selection workgroup for kernel `kind`.  Returns
// false when V does not fit at all.
enum class SelectKernel { kGreedy, kTopK, kFull, kRes };

bool plan_layout(const tsel_params *p, SelectKernel kind, tsel::SelectArgs *a,
                 size_t *lds_bytes) {
  const int32_t V = p->vocab;
  const int32_t mw = (V + 31) / 32;
  const size_t mask_bytes = align16((size_t)mw * 4);
  const size_t base = 2 * mask_bytes;
  // the kill table (8 or 4 kill bits -> per-word masks); the resident kernel
  // builds its masks with ALU operations and keeps a list offset per mask
  // word instead
  const size_t lut = kind == SelectKernel::kRes ? 0 : (size_t)(p->dtype == TSEL_BF16 ? 256 : 16) * 16;
  const size_t radix = 1024;
  const size_t woff = kind == SelectKernel::kRes ? align16(2 * (size_t)mw) : 0;
  const size_t budget = (size_t)tsel::kSelectMaxDynLds;
  const size_t fixed = base + lut + radix + woff;
  const size_t min_list = 8 * 64;
  if (fixed + min_list > budget) return false;
  // every distinct history id plus the row's tail elements; a multiple of 4
  // so that the value array stays 16-byte aligned
  size_t lcap = (size_t)std::min<int64_t>(std::max<int64_t>(p->hist_stride, 0), V) + 8;
  lcap = std::min<size_t>((lcap + 3) & ~size_t(3), kMaxList);
  int32_t nb = 0, ccap = 0, mant = 0, tcap = 0, vb = 0;
  size_t area = 0;
  if (kind == SelectKernel::kTopK) {
    tcap = 2048;
    while (tcap > 256 && fixed + 24 * (size_t)tcap + 8 * lcap > budget) tcap /= 2;
    area = 24 * (size_t)tcap;
  } else if (kind == SelectKernel::kRes) {
    // two histogram copies (the second, after folding, holds the collect
    // buffer), the head buffer (512 keys and masses), the ordered sub-bin
    mant = 6;
    auto need = [&]() {
      nb = (tsel::kBinBelow + tsel::kBinAbove) << mant;
      ccap = (int32_t)std::min<size_t>(4096, (8 * (size_t)nb) / 12);
      return 16 * (size_t)nb + 16 + 12 * 512 + 12 * (size_t)tsel::kGatherCap;
    };
    area = need();
    while (mant > 3 && fixed + area + 8 * lcap > budget) {
      --mant;
      area = need();
    }
  } else if (kind == SelectKernel::kFull) {
    // bf16 rows: two copies of the value bins of the streamed histogram pass,
    // when they fit beside the rest (else that pass counts by mass)
    for (int with = p->dtype == TSEL_BF16 ? 1 : 0; with >= 0; --with) {
      mant = 6;
      ccap = 4096;
      const size_t vbins = with ? 2 * 4 * (size_t)tsel::kVStride : 0;
      auto need = [&]() {
        nb = (tsel::kBinBelow + tsel::kBinAbove) << mant;
        // collected (key, mass) pairs, then room to order one sub-bin
        return 8 * (size_t)nb + 12 * (size_t)ccap + 12 * (size_t)tsel::kGatherCap + vbins;
      };
      area = need();
      while ((mant > 3 || ccap > 256) && fixed + area + 8 * lcap > budget) {
        if (mant > 3) --mant; else ccap /= 2;
        area = need();
      }
      vb = with;
      if (fixed + area + min_list <= budget) break;
    }
  }
  if (fixed + area + min_list > budget) return false;
  if (fixed + area + 8 * lcap > budget)  // rows that overflow apply penalties densely
    lcap = ((budget - fixed - area) / 8) & ~size_t(3);
  a->mw = mw;
  a->lcap = (int32_t)lcap;
  a->nb = nb;
  a->ccap = ccap;
  a->bin_mant = mant;
  a->tcap = tcap;
  a->vbins = vb;
  a->off_smask = (uint32_t)mask_bytes;
  a->off_list_id = (uint32_t)base;
  a->off_list_val = (uint32_t)(base + 4 * lcap);
  a->off_lut = (uint32_t)align16(base + 8 * lcap);
  a->off_rhist = (uint32_t)(a->off_lut + lut);
  a->off_woff = (uint32_t)(a->off_rhist + radix);
  a->off_area = (uint32_t)(a->off_woff + woff);
  *lds_bytes = a->off_area + area;
  return *lds_bytes <= budget;
}

// On-chip layout of the value-bin resident kernel (bf16): the histogram
// copies from byte 0 (the kernel computes bin offsets from there in 16
// bits), then the kill and seen masks, the list (seen ids, then the listed
// near-zero scores) and the list offset of every mask word.
bool plan_vres(const tsel_params *p, int res, tsel::SelectArgs *a, size_t *lds_bytes) {
  const int32_t V = p->vocab;
  const int32_t mw = (V + 31) / 32;
  // the kill and seen masks run to one byte per chunk slot of the registers,
  // the list offsets to one per four slots
  const size_t slots = (size_t)res * tsel::kSelectThreads;
  const size_t kmask_bytes = align16(std::max<size_t>((size_t)mw * 4, slots));
  const size_t smask_bytes = kmask_bytes;
  const size_t woff = align16(std::max<size_t>(2 * (size_t)mw, slots / 2));
  const size_t budget = (size_t)tsel::kVMaxDynLds;
  size_t off = align16((size_t)tsel::kVHistBytes);
  const size_t fixed = off + kmask_bytes + smask_bytes + woff + tsel::kVSharedBytes;
  size_t lcap = (size_t)std::min<int64_t>(std::max<int64_t>(p->hist_stride, 0), V) + 8;
  lcap = std::min<size_t>((lcap + 3) & ~size_t(3), kMaxList);
  if (fixed + 8 * (64 + (size_t)tsel::kZoneCap) > budget) return false;
  if (fixed + 8 * (lcap + tsel::kZoneCap) > budget)  // longer histories: the streamed path
    lcap = ((budget - fixed) / 8 - tsel::kZoneCap) & ~size_t(3);
  const size_t lall = lcap + tsel::kZoneCap;
  a->mw = mw;
  a->lcap = (int32_t)lcap;
  a->nb = tsel::kVBins;
  a->ccap = 0;
  a->bin_mant = 0;
  a->tcap = 0;
  a->vbins = 0;
  a->off_kmask = (uint32_t)off;
  off += kmask_bytes;
  a->off_smask = (uint32_t)off;
  off += smask_bytes;
  a->off_list_id = (uint32_t)off;
  off += 4 * lall;
  a->off_list_val = (uint32_t)off;
  off += 4 * lall;
  a->off_woff = (uint32_t)align16(off);
  off = a->off_woff + woff;
  a->off_sh = (uint32_t)align16(off);
  off = a->off_sh + tsel::kVSharedBytes;
  a->off_lut = a->off_rhist = a->off_area = 0;  // unused here
  *lds_bytes = off;
  return off <= budget;
}

// Chunks of 16 bytes per lane that hold a whole row in registers on the full
// path (0: the row is re-read from memory on each pass).
int resident_chunks(const tsel_params *p) {
  const int epc = p->dtype == TSEL_BF16 ? 8 : 4;
  const int64_t chunks = (p->vocab + epc - 1) / epc;
  for (int r : {4, 8, 16})
    if (chunks <= (int64_t)r * tsel::kSelectThreads) return r;
  return 0;
}

}  // namespace

extern "C" {

const char *tsel_status_string(tsel_status s) {
  switch (s) {
    case TSEL_OK: return "ok";
    case TSEL_ERR_INVALID_ARG: return "invalid argument";
    case TSEL_ERR_UNSUPPORTED: return "unsupported argument combination";
    case TSEL_ERR_LAUNCH: return "kernel launch failed";
    case TSEL_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

tsel_status tsel_validate_params(const tsel_params *params, int32_t sampling_uniforms_given) {
  return check_params(params, sampling_uniforms_given != 0);
}

// The rows and the processors' settings of p as kernel arguments (the
// warpers off).
static tsel::SelectArgs proc_args(const tsel_params *params, const void *logits,
                                  const int32_t *history, const int32_t *lens) {
  tsel::SelectArgs a{};
  const int64_t esize = params->dtype == TSEL_BF16 ? 2 : 4;
  a.logits = static_cast<const char *>(logits);
  a.row_bytes = params->logits_row_stride * esize;
  a.V = params->vocab;
  a.B = params->batch;
  a.dtype = params->dtype;
  a.hist = history;
  a.hist_stride = params->hist_stride;
  a.lens = lens;
  a.bad_mask = params->bad_words_mask;
  a.sup_mask = params->suppress_mask;
  a.begin_mask = params->begin_suppress_mask;
  a.rep = params->repetition_penalty;
  a.ngram = params->no_repeat_ngram_size;
  a.min_length = params->min_length;
  a.min_new = params->min_new_tokens;
  a.n_eos = params->n_eos;
  for (int i = 0; i < TSEL_MAX_EOS; ++i) a.eos[i] = i < params->n_eos ? params->eos_ids[i] : -1;
  a.forced_bos = params->forced_bos_token_id;
  a.forced_eos = params->forced_eos_token_id;
  a.temperature = 1.0f;
  a.top_p = 1.0f;
  return a;
}

// The kernel path one selection takes for the settings of p.  kTopK and
// kFull also finish the rows whose candidates overflow or whose history
// outgrows the resident list; every path but kGreedy and kRes computes the
// log-probabilities itself (the other two leave them to a pass over the
// final scores).
enum class Path { kGreedy, kVres, kRes, kTopK, kFull, kNone };

static Path select_path(const tsel_params *p) {
  tsel::SelectArgs probe{};
  size_t lds = 0;
  if (!p->do_sample)
    return plan_layout(p, SelectKernel::kGreedy, &probe, &lds) ? Path::kGreedy : Path::kNone;
  if (!plan_layout(p, SelectKernel::kFull, &probe, &lds)) return Path::kNone;
  const int res = resident_chunks(p);
  const int epc = p->dtype == TSEL_BF16 ? 8 : 4;
  const bool simple = p->top_k <= 0 && p->temperature == 1.0f && res > 0 && p->vocab >= epc;
  if (simple && p->dtype == TSEL_BF16 && plan_vres(p, res, &probe, &lds)) return Path::kVres;
  if (simple && plan_layout(p, SelectKernel::kRes, &probe, &lds)) return Path::kRes;
  if (p->top_k > 0 && plan_layout(p, SelectKernel::kTopK, &probe, &lds) &&
      std::min(p->top_k, p->vocab) * 4 <= probe.tcap)
    return Path::kTopK;
  return Path::kFull;
}

static bool fused_logprobs(Path path) { return path != Path::kGreedy && path != Path::kRes; }

// Rows of the workspace: the renormalized scores (fp32, a 16-byte aligned
// stride) when renormalize_logits is on, then the final scores a
// log-probability is taken over (fp32 [B, V]) when output_logprobs is and the
// selection's path leaves it to a pass over them.
static size_t renorm_stride(const tsel_params *p) { return ((size_t)p->vocab + 3) & ~size_t(3); }
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
static size_t renorm_bytes(const tsel_params *p) {
  return p->renormalize_logits ? align256((size_t)p->batch * renorm_stride(p) * 4) : 0;
}

// Rows whose byte stride is not a multiple of 16 are first copied into the
// workspace at the smallest stride that is (the kernels read rows in 16-byte
// units from 16-byte aligned starts).
static int64_t esize_of(const tsel_params *p) { return p->dtype == TSEL_BF16 ? 2 : 4; }
static bool needs_repack(const tsel_params *p) {
  return (p->logits_row_stride * esize_of(p)) % 16 != 0;
}
static int64_t repack_stride(const tsel_params *p) {
  const int64_t epu = 16 / esize_of(p);
  return ((int64_t)p->vocab + epu - 1) / epu * epu;
}
static size_t repack_bytes(const tsel_params *p) {
  return needs_repack(p) ? align256((size_t)p->batch * (size_t)repack_stride(p) * esize_of(p)) : 0;
}
// The repacked rows at the start of `ws` (when needed): *pr is params with
// their stride, *src their address; returns the workspace after them.
static char *repack_rows(const tsel_params *params, const void *logits, char *ws, tsel_params *pr,
                         const void **src, hipStream_t s, hipError_t *e) {
  *pr = *params;
  *src = logits;
  *e = hipSuccess;
  if (!needs_repack(params)) return ws;
  pr->logits_row_stride = repack_stride(params);
  *e = tsel::launch_repack(logits, params->dtype, params->logits_row_stride, ws,
                           pr->logits_row_stride, params->batch, params->vocab, s);
  *src = ws;
  return ws + repack_bytes(params);
}

// The params the selection itself sees: after renormalize_logits, fp32 rows
// with every processor switched off (the lengths still mark padding rows).
static tsel_params selection_params(const tsel_params *params) {
  tsel_params p = *params;
  if (!params->renormalize_logits) return p;
  p.dtype = TSEL_F32;
  p.logits_row_stride = (int64_t)renorm_stride(params);
  p.repetition_penalty = 1.0f;
  p.no_repeat_ngram_size = 0;
  p.bad_words_mask = p.suppress_mask = p.begin_suppress_mask = nullptr;
  p.min_length = p.min_new_tokens = 0;
  p.n_eos = 0;
  p.forced_bos_token_id = p.forced_eos_token_id = -1;
  p.renormalize_logits = 0;
  return p;
}

size_t tsel_process_select_workspace_size(const tsel_params *params) {
  if (!params || params->batch <= 0 || params->vocab < 1) return 0;
  size_t n = repack_bytes(params) + renorm_bytes(params);
  if (params->output_logprobs) {
    const tsel_params q = selection_params(params);
    if (!fused_logprobs(select_path(&q)))
      n += align256((size_t)params->batch * (size_t)params->vocab * 4);
  }
  return n;
}

// The kernels for one selection over `logits` with the settings of p (the
// arguments already checked); hipErrorNotSupported when V does not fit the
// on-chip layout.  out_logprobs is written only on the paths that compute it.
static hipError_t dispatch_select(const tsel_params *params, const void *logits,
                                  const int32_t *history, const int32_t *lens,
                                  const float *uniforms, int32_t *out_tokens, float *out_processed,
                                  float *out_logprobs, hipStream_t s) {
  const Path path = select_path(params);
  if (path == Path::kNone) return hipErrorNotSupported;
  tsel::SelectArgs a = proc_args(params, logits, history, lens);
  a.uniforms = uniforms;
  a.out_tokens = out_tokens;
  a.out_processed = out_processed;
  a.out_logprobs = fused_logprobs(path) ? out_logprobs : nullptr;
  a.do_sample = params->do_sample ? 1 : 0;
  a.temperature = params->temperature;
  a.top_k = params->top_k;
  a.top_p = params->top_p;
  size_t lds = 0;
  if (path == Path::kGreedy) {  // greedy: the warpers do not apply
    a.temperature = 1.0f;
    a.top_k = 0;
    a.top_p = 1.0f;
    plan_layout(params, SelectKernel::kGreedy, &a, &lds);
    return tsel::launch_greedy(a, lds, s);
  }
  plan_layout(params, SelectKernel::kFull, &a, &lds);
  const int res = resident_chunks(params);
  const int64_t most_seen = std::min<int64_t>(std::max(params->hist_stride, 0), a.V);
  tsel::SelectArgs r = a;
  size_t rlds = 0;
  hipError_t e = hipSuccess;
  switch (path) {
    case Path::kVres:
      // bf16 row held in registers, one histogram bin per bf16 value; rows
      // with more distinct seen ids than the list holds are left pending
      // for the streamed path
      plan_vres(params, res, &r, &rlds);
      e = tsel::launch_vres(r, res, rlds, s);
      if (e == hipSuccess && r.lcap < most_seen) e = tsel::launch_full(a, res, lds, s, 1);
      break;
    case Path::kRes:
      // Row held in registers.  A row with more distinct seen ids than the
      // on-chip list holds is left pending for the streamed path.
      plan_layout(params, SelectKernel::kRes, &r, &rlds);
      e = tsel::launch_res(r, res, rlds, s);
      if (e == hipSuccess && r.lcap < most_seen) e = tsel::launch_full(a, res, lds, s, 1);
      break;
    case Path::kTopK: {
      // Candidate-buffer pass; a row whose ties overflow it runs the full
      // path in the same workgroup, with that path's layout.
      tsel::SelectArgs t = a;
      size_t tlds = 0;
      plan_layout(params, SelectKernel::kTopK, &t, &tlds);
      e = tsel::launch_topk(t, a, std::max(tlds, lds), s);
      break;
    }
    default:
      e = tsel::launch_full(a, res, lds, s, 0);
  }
  return e;
}

tsel_status tsel_process_select(const void *logits, const int32_t *history, const int32_t *lens,
                                const tsel_params *params, const float *uniforms,
                                int32_t *out_tokens, float *out_processed, float *out_logprobs,
                                void *workspace, size_t workspace_bytes, void *stream) {
  tsel_status st = check_params(params, uniforms != nullptr);
  if (st != TSEL_OK) return st;
  if ((out_logprobs != nullptr) != (params->output_logprobs != 0)) return TSEL_ERR_INVALID_ARG;
  if (params->batch == 0) return TSEL_OK;
  if (!logits || !lens || !out_tokens) return TSEL_ERR_INVALID_ARG;
  if (!history && params->hist_stride > 0) return TSEL_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0) return TSEL_ERR_UNSUPPORTED;
  const size_t need = tsel_process_select_workspace_size(params);
  if (need > 0 && (!workspace || workspace_bytes < need)) return TSEL_ERR_WORKSPACE;
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TSEL_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  tsel_params pr;
  const void *src;
  hipError_t e;
  char *ws = repack_rows(params, logits, static_cast<char *>(workspace), &pr, &src, s, &e);
  if (e != hipSuccess) return TSEL_ERR_LAUNCH;
  params = &pr;
  logits = src;
  const tsel_params p = selection_params(params);
  if (params->renormalize_logits) {
    // the processors and the log-softmax into fp32 rows; the selection then
    // reads those with every processor switched off (the lengths still mark
    // padding rows)
    tsel::SelectArgs ra = proc_args(params, logits, history, lens);
    size_t lds = 0;
    if (!plan_layout(params, SelectKernel::kGreedy, &ra, &lds)) return TSEL_ERR_UNSUPPORTED;
    e = tsel::launch_renorm(ra, lds, reinterpret_cast<float *>(ws), (int64_t)renorm_stride(params), s);
    if (e != hipSuccess) return TSEL_ERR_LAUNCH;
    src = ws;
    ws += renorm_bytes(params);
  }
  // log-probabilities: from the selection kernels, or from a pass over the
  // final scores (into the workspace when the caller does not want them)
  const bool post = out_logprobs && !fused_logprobs(select_path(&p));
  float *proc = out_processed;
  if (post && !proc) proc = reinterpret_cast<float *>(ws);
  e = dispatch_select(&p, src, history, lens, uniforms, out_tokens, proc, out_logprobs, s);
  if (e == hipErrorNotSupported) return TSEL_ERR_UNSUPPORTED;  // (a layout that does not fit)
  if (e == hipSuccess && post)
    e = tsel::launch_logprob(proc, params->vocab, params->batch, params->vocab, out_tokens,
                             out_logprobs, s);
  return e == hipSuccess ? TSEL_OK : TSEL_ERR_LAUNCH;
}

// tsel_verify_select: the position rows' histories, lengths and tokens,
// then the selection's own workspace.
static tsel_params vsel_params(const tsel_params *p, int32_t k) {
  tsel_params q = *p;
  q.batch = p->batch * (k + 1);
  q.hist_stride = std::max(p->hist_stride, 0) + k;
  return q;
}
static size_t vsel_rows_bytes(const tsel_params *p, int32_t k) {
  const size_t R = (size_t)p->batch * (size_t)(k + 1);
  const size_t H2 = (size_t)std::max(p->hist_stride, 0) + (size_t)k;
  return align256(R * H2 * 4) + align256(R * 3 * 4) + align256(R * 4);
}

size_t tsel_verify_select_workspace_size(const tsel_params *params, int32_t k) {
  if (!params || params->batch <= 0 || params->vocab < 1 || k < 0) return 0;
  const tsel_params q = vsel_params(params, k);
  return vsel_rows_bytes(params, k) + tsel_process_select_workspace_size(&q);
}

tsel_status tsel_verify_select(const void *logits, const int32_t *history, const int32_t *lens,
                               const tsel_params *params, int32_t k, const int32_t *candidates,
                               const float *uniforms, int32_t *out_n_match, int32_t *out_tokens,
                               int32_t *out_next, int32_t *out_k, void *workspace,
                               size_t workspace_bytes, void *stream) {
  if (k < 0) return TSEL_ERR_INVALID_ARG;
  tsel_status st = check_params(params, uniforms != nullptr);
  if (st != TSEL_OK) return st;
  if (params->output_logprobs) return TSEL_ERR_INVALID_ARG;
  if (params->batch == 0) return TSEL_OK;
  if (!logits || !lens || !out_n_match || !out_tokens || !out_next || !out_k)
    return TSEL_ERR_INVALID_ARG;
  if (k > 0 && !candidates) return TSEL_ERR_INVALID_ARG;
  if (!history && params->hist_stride > 0) return TSEL_ERR_INVALID_ARG;
  if (k > tsel::kMaxVerifyK) return TSEL_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0) return TSEL_ERR_UNSUPPORTED;
  if ((int64_t)params->batch * (k + 1) > (int64_t)INT32_MAX / 4) return TSEL_ERR_UNSUPPORTED;
  const size_t need = tsel_verify_select_workspace_size(params, k);
  if (!workspace || workspace_bytes < need) return TSEL_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TSEL_ERR_UNSUPPORTED;
  const tsel_params q = vsel_params(params, k);
  {  // (the position rows must fit the selection too)
    tsel::SelectArgs probe{};
    size_t lds = 0;
    if (!plan_layout(&q, params->do_sample ? SelectKernel::kFull : SelectKernel::kGreedy, &probe,
                     &lds))
      return TSEL_ERR_UNSUPPORTED;
  }
  const size_t R = (size_t)q.batch;
  char *ws = static_cast<char *>(workspace);
  int32_t *hist2 = reinterpret_cast<int32_t *>(ws);
  ws += align256(R * (size_t)q.hist_stride * 4);
  int32_t *lens2 = reinterpret_cast<int32_t *>(ws);
  ws += align256(R * 3 * 4);
  int32_t *sel = reinterpret_cast<int32_t *>(ws);
  ws += align256(R * 4);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = tsel::launch_vsel_expand(history, params->hist_stride, lens, params->batch, k,
                                          candidates, hist2, q.hist_stride, lens2, s);
  if (e != hipSuccess) return TSEL_ERR_LAUNCH;
  st = tsel_process_select(logits, hist2, lens2, &q, uniforms, sel, nullptr, nullptr, ws,
                           workspace_bytes - (size_t)(ws - static_cast<char *>(workspace)), stream);
  if (st != TSEL_OK) return st;
  e = tsel::launch_vsel_match(sel, params->batch, k, candidates, out_n_match, out_tokens, out_next,
                              out_k, s);
  return e == hipSuccess ? TSEL_OK : TSEL_ERR_LAUNCH;
}

int32_t tsel_beam_width(int32_t num_beams, int32_t n_eos) {
  if (num_beams < 1 || n_eos < 0) return 0;
  const int64_t k = (int64_t)std::max<int64_t>(2, 1 + (int64_t)n_eos) * num_beams;
  return k > INT32_MAX ? 0 : (int32_t)k;
}

size_t tsel_beam_step_workspace_size(const tsel_params *params, int32_t num_beams) {
  if (!params || params->batch <= 0 || num_beams < 1) return 0;
  const int32_t K = tsel_beam_width(num_beams, std::max(params->n_eos, 0));
  return repack_bytes(params) + align256((size_t)params->batch * (size_t)K * 8);
}

tsel_status tsel_beam_step(const void *logits, const int32_t *history, const int32_t *lens,
                           const tsel_params *params, int32_t num_beams,
                           const float *beam_scores, int32_t first_step, float *out_scores,
                           int32_t *out_beams, int32_t *out_tokens, void *workspace,
                           size_t workspace_bytes, void *stream) {
  tsel_status st = check_params(params, false);
  if (st != TSEL_OK) return st;
  if (params->do_sample || params->renormalize_logits || params->output_logprobs)
    return TSEL_ERR_INVALID_ARG;
  if (num_beams < 1 || params->batch % num_beams != 0) return TSEL_ERR_INVALID_ARG;
  if (num_beams > tsel::kMaxBeams) return TSEL_ERR_UNSUPPORTED;
  if ((int64_t)num_beams * params->vocab > (int64_t)UINT32_MAX) return TSEL_ERR_UNSUPPORTED;
  if (tsel::beam_rows_lds(params->vocab) > (size_t)tsel::kSelectMaxDynLds)
    return TSEL_ERR_UNSUPPORTED;
  if (params->batch == 0) return TSEL_OK;
  if (!logits || !lens || !beam_scores || !out_scores || !out_beams || !out_tokens)
    return TSEL_ERR_INVALID_ARG;
  if (!history && params->hist_stride > 0) return TSEL_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0) return TSEL_ERR_UNSUPPORTED;
  const size_t need = tsel_beam_step_workspace_size(params, num_beams);
  if (!workspace || workspace_bytes < need) return TSEL_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TSEL_ERR_UNSUPPORTED;
  tsel_params pr;
  const void *src;
  hipError_t e;
  char *ws = repack_rows(params, logits, static_cast<char *>(workspace), &pr, &src,
                         static_cast<hipStream_t>(stream), &e);
  if (e != hipSuccess) return TSEL_ERR_LAUNCH;
  tsel::BeamArgs a{};
  a.s = proc_args(&pr, src, history, lens);
  a.nb = num_beams;
  a.width = tsel_beam_width(num_beams, params->n_eos);
  a.first_step = first_step ? 1 : 0;
  a.beam_scores = beam_scores;
  a.row_keys = reinterpret_cast<uint64_t *>(ws);
  a.out_scores = out_scores;
  a.out_beams = out_beams;
  a.out_tokens = out_tokens;
  e = tsel::launch_beam(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TSEL_OK : TSEL_ERR_LAUNCH;
}

tsel_status tsel_mask_build(int32_t vocab, const int32_t *ids, int32_t n_ids, uint32_t *out_mask,
                            void *stream) {
  if (vocab < 1 || n_ids < 0 || !out_mask || (n_ids > 0 && !ids)) return TSEL_ERR_INVALID_ARG;
  hipError_t e =
      tsel::launch_mask_build(vocab, ids, n_ids, out_mask, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TSEL_OK : TSEL_ERR_LAUNCH;
}

tsel_status tsel_finish_step(int32_t batch, const int32_t *tokens, const int32_t *lens,
                             const int32_t *max_lengths, const int32_t *eos_ids, int32_t n_eos,
                             uint8_t *finished, int32_t *out_tokens, void *stream) {
  if (batch < 0 || n_eos < 0 || (n_eos > 0 && !eos_ids)) return TSEL_ERR_INVALID_ARG;
  if (batch > 0 && (!tokens || !lens || !max_lengths || !finished || !out_tokens))
    return TSEL_ERR_INVALID_ARG;
  if (n_eos > tsel::kMaxFinishEos) return TSEL_ERR_UNSUPPORTED;
  if (batch == 0) return TSEL_OK;
  hipError_t e = tsel::launch_finish(batch, tokens, lens, max_lengths, eos_ids, n_eos, finished,
                                     out_tokens, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TSEL_OK : TSEL_ERR_LAUNCH;
}

static size_t verify_partial_bytes(int32_t batch, int32_t k, int32_t vocab);

size_t tsel_verify_workspace_size(int32_t batch, int32_t k, int32_t vocab) {
  if (batch <= 0 || k < 0 || vocab < 1) return 0;
  return align16(verify_partial_bytes(batch, k, vocab));
}

// Host checks shared by both verify entry points (TSEL_OK to go on).
static tsel_status check_verify(const void *logits, int32_t dtype, int32_t batch, int32_t k,
                                int32_t vocab, int64_t row_stride, const int32_t *candidates,
                                const int32_t *out_n_match, const int32_t *out_tokens,
                                const int32_t *out_next, const int32_t *out_k) {
  if (batch < 0 || k < 0 || vocab < 1 || row_stride < vocab) return TSEL_ERR_INVALID_ARG;
  if (dtype != TSEL_F32 && dtype != TSEL_BF16) return TSEL_ERR_INVALID_ARG;
  if (batch == 0) return TSEL_OK;
  if (!logits || !out_n_match || !out_tokens || !out_next || !out_k) return TSEL_ERR_INVALID_ARG;
  if (k > 0 && !candidates) return TSEL_ERR_INVALID_ARG;
  if (k > tsel::kMaxVerifyK) return TSEL_ERR_UNSUPPORTED;
  const int64_t esize = dtype == TSEL_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0 || (row_stride * esize) % 16 != 0)
    return TSEL_ERR_UNSUPPORTED;
  if ((int64_t)batch * (k + 1) > 65535) return TSEL_ERR_UNSUPPORTED;  // grid y limit
  return TSEL_OK;
}

static size_t verify_partial_bytes(int32_t batch, int32_t k, int32_t vocab) {
  const int Smax = std::max(tsel::verify_chunks(vocab, TSEL_F32), tsel::verify_chunks(vocab, TSEL_BF16));
  return (size_t)batch * (size_t)(k + 1) * (size_t)Smax * 8;
}

tsel_status tsel_verify(const void *logits, int32_t dtype, int32_t batch, int32_t k,
                        int32_t vocab, int64_t row_stride, const int32_t *candidates,
                        int32_t *out_n_match, int32_t *out_tokens, int32_t *out_next,
                        int32_t *out_k, void *workspace, size_t workspace_bytes, void *stream) {
  tsel_status st = check_verify(logits, dtype, batch, k, vocab, row_stride, candidates,
                                out_n_match, out_tokens, out_next, out_k);
  if (st != TSEL_OK || batch == 0) return st;
  const size_t need = tsel_verify_workspace_size(batch, k, vocab);
  if (!workspace || workspace_bytes < need) return TSEL_ERR_WORKSPACE;
  const int64_t esize = dtype == TSEL_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(workspace) % 8 != 0) return TSEL_ERR_UNSUPPORTED;
  const int S = tsel::verify_chunks(vocab, dtype);
  hipError_t e = tsel::launch_verify(logits, dtype, batch, k, vocab, row_stride * esize, S,
                                     candidates, out_n_match, out_tokens, out_next, out_k,
                                     static_cast<uint64_t *>(workspace),
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TSEL_OK : TSEL_ERR_LAUNCH;
}

tsel_status tsel_verify_noalloc(const void *logits, int32_t dtype, int32_t batch, int32_t k,
                                int32_t vocab, int64_t row_stride, const int32_t *candidates,
                                int32_t *out_n_match, int32_t *out_tokens, int32_t *out_next,
                                int32_t *out_k, void *stream) {
  tsel_status st = check_verify(logits, dtype, batch, k, vocab, row_stride, candidates,
                                out_n_match, out_tokens, out_next, out_k);
  if (st != TSEL_OK || batch == 0) return st;
  if (tsel_verify_workspace_size(batch, k, vocab) > tsel::kNoAllocScratchBytes)
    return TSEL_ERR_UNSUPPORTED;
  const int64_t esize = dtype == TSEL_BF16 ? 2 : 4;
  hipError_t e = tsel::launch_verify_noalloc(
      logits, dtype, batch, k, vocab, row_stride * esize, tsel::verify_chunks(vocab, dtype),
      candidates, out_n_match, out_tokens, out_next, out_k, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TSEL_OK : TSEL_ERR_LAUNCH;
}

}  // extern "C"
