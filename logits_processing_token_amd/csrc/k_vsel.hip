// k_vsel.hip -- verification of assistant drafts with the token selection
// method of the step ("Assisted Generation: a new direction toward
// low-latency text generation", "Greedy decoding with assisted generation",
// step 3: ".argmax() for greedy search or .multinomial() for sampling", and
// "Sample with assisted generation").
//
// Position j of batch row b was computed by the model after the row's
// history and the drafts 0..j-1, so the selection of that position sees the
// history extended by those drafts and the length L + j (the length rules
// move with it).  The B * (k+1) positions become rows of one selection:
//  * k_vsel_expand writes each position row's history (the row's ids, then
//    its first j drafts) and lengths into the workspace;
//  * the selection kernels run over them (their logits rows are the
//    positions' own, at the caller's stride), one uniform per position;
//  * k_vsel_match compares the drafts with the selected tokens left to
//    right (steps 4-6: the matches, the first divergent token, next k).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsel_internal.hpp"

namespace tsel {

constexpr int kExpandThreads = 256;

// One workgroup per position row r = b * (k+1) + j.
__global__ __launch_bounds__(kExpandThreads) void k_vsel_expand(
    const int32_t *hist, int32_t hist_stride, const int32_t *lens, int32_t B, int32_t k,
    const int32_t *cand, int32_t *hist2, int32_t hist2_stride, int32_t *lens2) {
  const int r = blockIdx.x, R = B * (k + 1);
  const int b = r / (k + 1), j = r % (k + 1);
  const int L = lens[b];
  int32_t *dst = hist2 + (int64_t)r * hist2_stride;
  const int32_t *src = hist + (int64_t)b * hist_stride;
  const int Lc = min(max(L, 0), hist_stride);  // (ids past the stride are not the row's)
  for (int i = threadIdx.x; i < Lc; i += kExpandThreads) dst[i] = src[i];
  if (L > 0)
    for (int i = threadIdx.x; i < j; i += kExpandThreads) dst[Lc + i] = cand[(int64_t)b * k + i];
  if (threadIdx.x == 0) {
    lens2[r] = L > 0 ? Lc + j : 0;  // (a padding row stays one)
    lens2[R + r] = lens[B + b];
    lens2[2 * R + r] = lens[2 * B + b];
  }
}

// One thread per batch row.
__global__ __launch_bounds__(256) void k_vsel_match(const int32_t *sel, int32_t B, int32_t k,
                                                    const int32_t *cand, int32_t *n_match,
                                                    int32_t *tokens, int32_t *next,
                                                    int32_t *k_out) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int32_t *s = sel + (int64_t)b * (k + 1);
  int n = 0;
  while (n < k && cand[(int64_t)b * k + n] == s[n]) ++n;  // (stops at the first mismatch)
  for (int j = 0; j <= k; ++j) tokens[(int64_t)b * (k + 1) + j] = j <= n ? s[j] : -1;
  n_match[b] = n;
  next[b] = s[n];
  k_out[b] = n == k ? k + 2 : (k - 1 > 1 ? k - 1 : 1);
}

hipError_t launch_vsel_expand(const int32_t *hist, int32_t hist_stride, const int32_t *lens,
                              int32_t B, int32_t k, const int32_t *cand, int32_t *hist2,
                              int32_t hist2_stride, int32_t *lens2, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_vsel_expand, dim3(B * (k + 1)), dim3(kExpandThreads), 0, s, hist,
                     hist_stride, lens, B, k, cand, hist2, hist2_stride, lens2);
  return hipGetLastError();
}

hipError_t launch_vsel_match(const int32_t *sel, int32_t B, int32_t k, const int32_t *cand,
                             int32_t *n_match, int32_t *tokens, int32_t *next, int32_t *k_out,
                             hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_vsel_match, dim3((B + 255) / 256), dim3(256), 0, s, sel, B, k, cand,
                     n_match, tokens, next, k_out);
  return hipGetLastError();
}

}  // namespace tsel
