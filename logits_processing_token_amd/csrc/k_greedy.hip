// k_greedy.hip -- greedy token selection: the argmax of the processed scores
// of each row (lowest id among equal maxima), one coalesced pass.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k_select_common.hpp"

namespace tsel {

// =========================================================================
// k_greedy: argmax of the processed scores (lowest id among equal maxima).
template <int DT>
__global__ __launch_bounds__(NT, 1) void k_greedy(SelectArgs a) {
  constexpr int EPC = Elem<DT>::EPC;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RowShared sh;
  const Lds s = carve(a, smem);
  const int tid = threadIdx.x, row = blockIdx.x, V = a.V;
  RowInfo ri;
  if (row_prologue(a, row, ri)) return;
  stage_row<DT>(a, row, ri, s, sh);
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  float *outp = a.out_processed ? a.out_processed + (int64_t)row * V : nullptr;
  const bool dense_pen = sh.dense_pen != 0;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  stream_row<DT>(a, rowp, s, dense_pen, [&](int v, float x) {
    if (x > bv) { bv = x; bi = v; }  // ids rise within a lane: the first maximum stays
    if (outp) outp[v] = x;
  });
  uint64_t key = bi == 0x7FFFFFFF ? 0ull : sel_key(bv, (uint32_t)bi);
  const int n_list = sh.n_list;
  for (int i = tid; i < n_list; i += NT) {
    const uint64_t k2 = sel_key(s.list_val[i], (uint32_t)s.list_id[i]);
    key = k2 > key ? k2 : key;
  }
  key = block_max_u64<NT>(key, sh.red_u64);
  if (tid == 0) a.out_tokens[row] = key == 0ull ? 0 : (int)key_index(key);
  if (outp) {
    for (int v = (V / EPC) * EPC + tid; v < V; v += NT) outp[v] = -INFINITY;
    __syncthreads();
    for (int i = tid; i < n_list; i += NT) outp[s.list_id[i]] = s.list_val[i];
  }
}

template <int DT>
hipError_t launch_greedy_t(const SelectArgs &a, size_t lds, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};  // devices where the limit is raised
  const void *fn = reinterpret_cast<const void *>(&k_greedy<DT>);
  if (hipError_t e = ensure_dyn_lds(fn, (int)kSelectMaxDynLds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(k_greedy<DT>, dim3(a.B), dim3(NT), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_greedy(const SelectArgs &a, size_t lds, hipStream_t st) {
  return a.dtype == 1 ? launch_greedy_t<1>(a, lds, st) : launch_greedy_t<0>(a, lds, st);
}

}  // namespace tsel
