// tsel_internal.hpp -- launch descriptors shared by the C-ABI layer
// (tsel_api.cpp) and the kernels.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace tsel {

// Raises a kernel's dynamic LDS limit on the current device the first time
// it launches there.  `done` holds one bit per device id below 64 (higher
// ids set the attribute on every launch); two threads racing on a first
// launch both set the same value, which is harmless.
inline hipError_t ensure_dyn_lds(const void *fn, int bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

constexpr int kSelectThreads = 1024;        // one workgroup (16 wave64s) per row
constexpr int kLdsBytes = 160 * 1024;       // LDS of one gfx950 compute unit
constexpr int kSelectStaticLds = 12288;     // upper bound of the kernels' static LDS
constexpr int kSelectMaxDynLds = kLdsBytes - kSelectStaticLds;
constexpr int kVMaxDynLds = kLdsBytes;     // the value-bin kernel has no static LDS
constexpr int kMaxVerifyK = 1023;           // drafts per row a verify call accepts

// Mass histogram of the full path: bins cover masses from 2^-kBinBelow to
// 2^kBinAbove relative to the reference, 2^bin_mant bins per binade.
constexpr int kBinBelow = 50;
constexpr int kBinAbove = 16;
constexpr int kGatherCap = 256;           // elements of one mass sub-bin ordered on chip
constexpr float kRefSlack = 2.0f;           // reference = first-chunk max + this (nats)
constexpr int kKeepBelow = 11;              // binades under the reference whose elements the
                                            // streamed histogram pass keeps on chip

// Value-bin resident kernel (bf16 rows): one bin per bf16 value.
constexpr int kVBins = 4032;                // bins; bin 0 takes the dropped scores
constexpr int kVStride = kVBins + 8;        // words between histogram copies (bank offset 8)
constexpr int kVCopies = 4;                 // histogram copies, by lane
constexpr int kZoneExp = 8;                 // scores below 2^-kZoneExp in magnitude share a bin
constexpr float kDropNats = 36.0f;          // bins start this far below the first chunks' max
constexpr int kZoneCap = 512;               // near-zero scores listed one by one
constexpr int kVPipe = 4;                   // chunks in flight per lane while counting
constexpr int kVHistBytes = kVCopies * kVStride * 4;  // the copies, from LDS byte 0
constexpr int kVMassOff = kVStride * 4;     // after the fold: per-bin masses (doubles)
constexpr int kVViewOff = kVMassOff + kVBins * 8;     // then the ordered view of one bin
constexpr int kVRowSharedBytes = 1024;      // the row's shared scalars, then the kernel's own
constexpr int kVSharedBytes = 4096;
constexpr int kVAboveOff = kVViewOff + 24 * kGatherCap;  // then one double per thread
constexpr int kGatherCap2 = 64;            // individuals of a second view (the predicted draw's)
constexpr int kVView2Off = kVAboveOff + 8 * kSelectThreads;  // then that view
static_assert(kVView2Off + 24 * kGatherCap2 <= kVHistBytes, "beyond the copies");
static_assert((kVCopies - 1) * kVStride * 4 + (kVBins - 1) * 4 < 65536,
              "bin offsets are computed in 16 bits");


// Arguments of the selection kernels (passed by value).
struct SelectArgs {
  const char *logits;
  int64_t row_bytes;        // bytes between rows
  int32_t V, B, dtype;
  const int32_t *hist;
  int32_t hist_stride;
  const int32_t *lens;      // [3][B]
  const float *uniforms;
  int32_t *out_tokens;
  float *out_processed;
  float *out_logprobs;      // the token's log-probability, when the kernel computes it
  const uint32_t *bad_mask, *sup_mask, *begin_mask;
  float rep;
  int32_t ngram;
  int32_t min_length, min_new;
  int32_t n_eos;
  int32_t eos[8];
  int32_t forced_bos, forced_eos;
  int32_t do_sample;
  float temperature;
  int32_t top_k;
  float top_p;
  // on-chip layout (kill mask at byte 0) and capacities
  int32_t mw;               // mask words: ceil(V / 32)
  int32_t lcap;             // sparse list capacity
  int32_t nb, ccap;         // full path: histogram bins, collect capacity
  int32_t bin_mant;         // full path: mantissa bits per bin
  int32_t tcap;             // top_k candidate capacity
  int32_t vbins;            // full path, bf16: the value bins fit on chip (else count by mass)
  uint32_t off_smask, off_list_id, off_list_val, off_lut, off_rhist, off_area;
  uint32_t off_woff;        // resident path: list offset of each thread's mask words
  uint32_t off_kmask;       // kill mask (0 but on the value-bin path)
  uint32_t off_sh;          // value-bin path: its shared scalars (no static LDS)
};

// One beam-search step: SelectArgs carries the processors' settings, B the
// beam rows (prompts * nb).
constexpr int kBeamThreads = 1024;
constexpr int kBeamSelBins = 8192;  // radix-select histogram (13-bit digits)
constexpr int kSelCap = 2048;       // keys ranked on chip at once
constexpr int kMaxBeams = 64;
struct BeamArgs {
  SelectArgs s;
  int32_t nb;                 // beams per prompt
  int32_t width;              // K, the candidates kept per prompt
  int32_t first_step;
  const float *beam_scores;   // [B]
  uint64_t *row_keys;         // workspace [B, K]: each row's best keys
  float *out_scores;          // [B / nb, K]
  int32_t *out_beams, *out_tokens;
};
size_t beam_rows_lds(int32_t V);
hipError_t launch_beam(const BeamArgs &a, hipStream_t s);

hipError_t launch_greedy(const SelectArgs &a, size_t lds, hipStream_t s);
// af: the full path's layout of the same call, for rows whose ties
// overflow the candidate buffer; lds covers both layouts
hipError_t launch_topk(const SelectArgs &a, const SelectArgs &af, size_t lds, hipStream_t s);
// pending != 0: only rows whose token an earlier kernel left as pending
hipError_t launch_full(const SelectArgs &a, int res, size_t lds, hipStream_t s, int pending);
// sampling without top_k at temperature 1, row held in `res` chunks per lane
hipError_t launch_res(const SelectArgs &a, int res, size_t lds, hipStream_t s);
// the same on bf16 rows with one histogram bin per bf16 value
hipError_t launch_vres(const SelectArgs &a, int res, size_t lds, hipStream_t s);

hipError_t launch_renorm(const SelectArgs &a, size_t lds, float *dst, int64_t dst_stride,
                         hipStream_t s);
hipError_t launch_logprob(const float *proc, int64_t stride, int32_t B, int32_t V,
                          const int32_t *tokens, float *out, hipStream_t s);

hipError_t launch_vsel_expand(const int32_t *hist, int32_t hist_stride, const int32_t *lens,
                              int32_t B, int32_t k, const int32_t *cand, int32_t *hist2,
                              int32_t hist2_stride, int32_t *lens2, hipStream_t s);
hipError_t launch_vsel_match(const int32_t *sel, int32_t B, int32_t k, const int32_t *cand,
                             int32_t *n_match, int32_t *tokens, int32_t *next, int32_t *k_out,
                             hipStream_t s);

hipError_t launch_verify(const void *logits, int32_t dtype, int32_t B, int32_t k, int32_t V,
                         int64_t row_bytes, int32_t chunks, const int32_t *cand,
                         int32_t *n_match, int32_t *tokens, int32_t *next, int32_t *k_out,
                         uint64_t *partials, hipStream_t s);
int verify_chunks(int32_t V, int32_t dtype);

// tsel_verify_noalloc: scratch of at most this many bytes per device, for
// device ids below kNoAllocDevices.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
constexpr int kNoAllocDevices = 64;
hipError_t launch_verify_noalloc(const void *logits, int32_t dtype, int32_t B, int32_t k,
                                 int32_t V, int64_t row_bytes, int32_t chunks,
                                 const int32_t *cand, int32_t *n_match, int32_t *tokens,
                                 int32_t *next, int32_t *k_out, hipStream_t s);

constexpr int kMaxFinishEos = 256;  // stop ids one end-of-step call takes
// Rows of V elements (dtype 1: bf16, else fp32) at src_stride elements apart
// copied to dst_stride elements apart (dst_stride * element size a multiple
// of 16; the destination 16-byte aligned), zeros after each row's V.
hipError_t launch_repack(const void *src, int32_t dtype, int64_t src_stride, void *dst,
                         int64_t dst_stride, int32_t rows, int32_t V, hipStream_t s);
hipError_t launch_finish(int32_t B, const int32_t *tokens, const int32_t *lens,
                         const int32_t *max_lengths, const int32_t *eos, int32_t n_eos,
                         uint8_t *finished, int32_t *out, hipStream_t s);
hipError_t launch_mask_build(int32_t V, const int32_t *ids, int32_t n, uint32_t *mask,
                             hipStream_t s);

}  // namespace tsel
