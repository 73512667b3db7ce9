// k_lsm.hip -- log-softmax steps around token selection ("Transmuter.
// Generation (transmuter v2.0.0)"): renormalize_logits, the processor that
// sits after the processors of the task and before temperature (module doc,
// processor order), and the token's log-probability, the log-softmax of the
// scores the step selects from at the token ("Log-probabilities").
//
// Both take the row's largest finite score m and S = sum of exp(x - m) over
// the finite scores in binary64 (exp on double): each thread folds its
// scores into a running (max, sum) pair, rescaling the sum when its maximum
// moves; the pairs are then joined over the workgroup at the row's maximum.
//
//  * k_renorm: the processed row (the processors of the module doc, staged
//    as for greedy selection) becomes (x - m) - ls with ls = log(S) rounded
//    once to binary32, two binary32 subtractions; -inf stays -inf.  It is
//    written as fp32 rows that the selection then reads with the processors
//    switched off.
//  * k_logprob: x[t] - m - log(S) in binary64, rounded once, over the final
//    scores a selection wrote; a row without a token (t < 0) gets the quiet
//    NaN with sign bit 0, and so does a row whose scores are all -inf.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k_select_common.hpp"

namespace tsel {

// =========================================================================
// k_renorm: processors, then the log-softmax of the row, into dst (fp32 rows
// of dst_stride elements).  Padding rows are left alone (the selection reads
// nothing of them); a forced row becomes -inf but for its forced id, 0.
template <int DT>
__global__ __launch_bounds__(NT, 1) void k_renorm(SelectArgs a, float *dst, int64_t dst_stride) {
  constexpr int EPC = Elem<DT>::EPC;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RowShared sh;
  const Lds s = carve(a, smem);
  const int tid = threadIdx.x, row = blockIdx.x, V = a.V;
  float *out = dst + (int64_t)row * dst_stride;
  RowInfo ri;
  row_lens(a, row, ri);
  ri.new_tokens = ri.L - ri.P;
  ri.begin_active =
      a.begin_mask != nullptr && ri.new_tokens == ((a.forced_bos >= 0 && ri.P == 1) ? 1 : 0);
  if (ri.L <= 0) return;
  int forced = -1;
  if (a.forced_bos >= 0 && ri.L == 1) forced = a.forced_bos;
  if (a.forced_eos >= 0 && ri.L == ri.M - 1) forced = a.forced_eos;
  if (forced >= 0) {
    bool alive = forced < V;
    if (alive && a.sup_mask && bit_of(a.sup_mask, forced)) alive = false;
    if (alive && ri.begin_active && bit_of(a.begin_mask, forced)) alive = false;
    // (a lone score 0: m = 0 and ls = log 1 = 0 leave it 0)
    for (int v = tid; v < V; v += NT) out[v] = (alive && v == forced) ? 0.0f : -INFINITY;
    return;
  }
  stage_row<DT>(a, row, ri, s, sh);
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  const bool dense_pen = sh.dense_pen != 0;
  const int n_list = sh.n_list;
  LseAcc acc;
  stream_row<DT>(a, rowp, s, dense_pen, [&](int, float x) { acc.add(x); });
  for (int i = tid; i < n_list; i += NT) acc.add(s.list_val[i]);
  float M;
  double S;
  lse_join<NT>(acc, sh.red_f32, sh.red_f64, &M, &S);
  const bool any = M > -INFINITY;
  const float lsf = any ? (float)log(S) : 0.0f;
  auto norm = [&](float x) { return (any && x > -INFINITY) ? (x - M) - lsf : x; };
  stream_row<DT>(a, rowp, s, dense_pen, [&](int v, float x) { out[v] = norm(x); });
  for (int v = (V / EPC) * EPC + tid; v < V; v += NT) out[v] = -INFINITY;
  __syncthreads();  // (the list's scores land after the stream's -inf)
  for (int i = tid; i < n_list; i += NT) out[s.list_id[i]] = norm(s.list_val[i]);
}

// =========================================================================
// k_logprob: the token's log-probability over the final scores of its row.
constexpr int kLpThreads = 256;

__global__ __launch_bounds__(kLpThreads) void k_logprob(const float *proc, int64_t stride, int V,
                                                        const int32_t *tokens, float *out) {
  __shared__ float rmax[kLpThreads / kWave];
  __shared__ double rsum[kLpThreads / kWave];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int t = tokens[row];
  const float qnan = lp_none();
  if (t < 0 || t >= V) {  // no token (a padding row)
    if (tid == 0) out[row] = qnan;
    return;
  }
  const float *x = proc + (int64_t)row * stride;
  LseAcc acc;
  for (int v = tid; v < V; v += kLpThreads) acc.add(x[v]);
  float M;
  double S;
  lse_join<kLpThreads>(acc, rmax, rsum, &M, &S);
  if (tid == 0)
    out[row] = M > -INFINITY ? (float)(((double)x[t] - (double)M) - log(S)) : qnan;
}

template <int DT>
static hipError_t launch_renorm_t(const SelectArgs &a, size_t lds, float *dst, int64_t dst_stride,
                                  hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};  // devices where the limit is raised
  const void *fn = reinterpret_cast<const void *>(&k_renorm<DT>);
  if (hipError_t e = ensure_dyn_lds(fn, (int)kSelectMaxDynLds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(k_renorm<DT>, dim3(a.B), dim3(NT), lds, st, a, dst, dst_stride);
  return hipGetLastError();
}

hipError_t launch_renorm(const SelectArgs &a, size_t lds, float *dst, int64_t dst_stride,
                         hipStream_t st) {
  return a.dtype == 1 ? launch_renorm_t<1>(a, lds, dst, dst_stride, st)
                      : launch_renorm_t<0>(a, lds, dst, dst_stride, st);
}

hipError_t launch_logprob(const float *proc, int64_t stride, int32_t B, int32_t V,
                          const int32_t *tokens, float *out, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_logprob, dim3(B), dim3(kLpThreads), 0, st, proc, stride, V, tokens, out);
  return hipGetLastError();
}

}  // namespace tsel
