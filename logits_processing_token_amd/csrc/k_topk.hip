// k_topk.hip -- sampling with a top_k: a running threshold filters each row
// into an on-chip candidate buffer; temperature, top_k, top_p and the
// inverse-CDF draw run exactly on the candidates.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k_select_common.hpp"

namespace tsel {

// =========================================================================
// k_topk: sampling with a top_k the candidate buffer holds.
template <int DT>
__global__ __launch_bounds__(NT, 1) void k_topk(SelectArgs a) {
  using E = Elem<DT>;
  constexpr int EPC = E::EPC;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RowShared sh;
  const Lds s = carve(a, smem);
  const int tid = threadIdx.x, row = blockIdx.x, V = a.V;
  RowInfo ri;
  if (row_prologue(a, row, ri)) return;
  stage_row<DT>(a, row, ri, s, sh);
  const char *rowp = a.logits + (int64_t)row * a.row_bytes;
  const bool dense_pen = sh.dense_pen != 0;
  const int n_list = sh.n_list;
  const float T = a.temperature;
  const int k_eff = min(a.top_k, V);
  const int NG = V / EPC;
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
  auto prep = [&](const uint4 &c, int g, int j) {
    float x = E::get(c, j);
    if (dense_pen && ((chunk_bits<DT>(s.smask, g) >> j) & 1u)) x = penalize(x, a.rep);
    return x;
  };
  // Threshold from the first chunk of every lane: the k-th largest alive
  // score among them, a lower bound of the row's.
  uint4 c0 = make_uint4(0u, 0u, 0u, 0u);
  if (tid < NG) c0 = kill_chunk<DT>(load16(rowp + (int64_t)tid * 16), tid, s);
  const uint32_t t0 = radix_kth_largest(
      [&](auto &&f) {
        if (tid < NG)
#pragma unroll
          for (int j = 0; j < EPC; ++j) {
            const float x = prep(c0, tid, j);
            if (x > -INFINITY) f(ordered_f32(x));
          }
      },
      k_eff, s.rhist, sh);
  if (tid == 0) sh.tau_x = pre_temperature_floor(t0 == 0u ? -INFINITY : unordered_f32(t0), T);
  __syncthreads();
  float flt = sh.tau_x;
  if (tid < NG)
#pragma unroll
    for (int j = 0; j < EPC; ++j) {
      const float x = prep(c0, tid, j);
      if (x > -INFINITY && x >= flt) append(tid * EPC + j, x);
    }
  for (int i = tid; i < n_list; i += NT)
    if (s.list_val[i] >= flt) append(s.list_id[i], s.list_val[i]);
  __syncthreads();
  for (int t0g = NT; t0g < NG && !sh.overflow; t0g += NT * U) {
    uint4 c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = t0g + tid + u * NT;
      if (g < NG) c[u] = load16(rowp + (int64_t)g * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = t0g + tid + u * NT;
      if (g < NG) {
        const uint4 ck = kill_chunk<DT>(c[u], g, s);
#pragma unroll
        for (int j = 0; j < EPC; ++j) {
          const float x = prep(ck, g, j);
          if (x > -INFINITY && x >= flt) append(g * EPC + j, x);
        }
      }
    }
    __syncthreads();
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
  if (sh.overflow) {  // k_full takes this row
    if (tid == 0) a.out_tokens[row] = kPending;
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
    if (tid == 0) sh.token = 0;
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
    if (tid == 0) {
      double W = 0.0;
      for (int j = 0; j < nk; ++j) W += w[j];
      int K = nk;
      if (a.top_p < 1.0f) {
        double run = 0.0;
        K = 0;
        for (int j = 0; j < nk; ++j) {
          if (run / W < (double)a.top_p) K = j + 1;
          run += w[j];
        }
      }
      double Wp = 0.0;
      for (int j = 0; j < K; ++j) Wp += w[j];
      const double target = (double)a.uniforms[row] * Wp;
      double C = 0.0;
      int pick = K - 1;
      for (int j = 0; j < K; ++j) {
        C += w[j];
        if (C > target) { pick = j; break; }
      }
      sh.token = (int)key_index(keys[pick]);
      sh.kcut = (K < nk) ? keys[K - 1] : 0ull;
    }
    __syncthreads();
    kcut = sh.kcut;
  }
  if (tid == 0) a.out_tokens[row] = sh.token;
  if (a.out_processed) write_processed<DT>(a, row, s, sh, nk == 0 ? INFINITY : t_y, kcut);
}

template <int DT>
hipError_t launch_topk_t(const SelectArgs &a, size_t lds, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};  // devices where the limit is raised
  const void *fn = reinterpret_cast<const void *>(&k_topk<DT>);
  if (hipError_t e = ensure_dyn_lds(fn, (int)kSelectMaxDynLds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(k_topk<DT>, dim3(a.B), dim3(NT), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_topk(const SelectArgs &a, size_t lds, hipStream_t st) {
  return a.dtype == 1 ? launch_topk_t<1>(a, lds, st) : launch_topk_t<0>(a, lds, st);
}

}  // namespace tsel
