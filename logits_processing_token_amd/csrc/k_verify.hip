// k_verify.hip -- greedy verification of assistant drafts over the
// [B, k+1, V] logits of the main model ("Assisted Generation: a new direction
// toward low-latency text generation", section "Greedy decoding with assisted
// generation", steps 3-6).
//
// Two launches.  k_verify_part: every (position row, vocabulary chunk) pair
// is one workgroup of 256 threads that streams its chunk once (16 bytes per
// lane per load) and writes the (score, id) argmax key of the chunk to the
// workspace.  k_verify_merge: one workgroup per batch row merges the chunk
// keys of its k+1 positions, counts the left-to-right matches, and writes
// the kept tokens, the next token and the next draft count.  The launch boundary
// orders the partial keys before the merge, so no workgroup needs a
// device-wide fence (on this GPU one writes back and invalidates the L2), and
// nothing in the workspace carries over from one call to the next.  Chunks
// keep the grid well above the 256 compute units even when B * (k+1) is
// small.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tsel_device.hpp"
#include "tsel_internal.hpp"

namespace tsel {

constexpr int VT = 256;   // threads per workgroup
constexpr int VCH = 8;    // 16-byte chunks per lane per workgroup

template <int DT>
__global__ __launch_bounds__(VT) void k_verify_part(const char *logits, int64_t row_bytes,
                                                    int V, int S, uint64_t *partials) {
  constexpr int EPC = DT == 1 ? 8 : 4;
  constexpr int CHUNK = VT * VCH * EPC;  // elements per workgroup
  __shared__ uint64_t red[VT / kWave];
  const int tid = threadIdx.x;
  const int s = blockIdx.x;       // chunk of the row
  const int r = blockIdx.y;       // position row b * (k+1) + j
  const char *rowp = logits + (int64_t)r * row_bytes;
  const int NG = V / EPC;
  const int e0 = s * CHUNK;

  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  uint4 c[VCH];
#pragma unroll
  for (int q = 0; q < VCH; ++q) {
    const int g = e0 / EPC + q * VT + tid;
    if (g < NG) c[q] = *reinterpret_cast<const uint4 *>(rowp + (int64_t)g * 16);
  }
#pragma unroll
  for (int q = 0; q < VCH; ++q) {
    const int g = e0 / EPC + q * VT + tid;
    if (g < NG) {
      const uint32_t w[4] = {c[q].x, c[q].y, c[q].z, c[q].w};
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        const float x = DT == 1 ? ((j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]))
                                : __uint_as_float(w[j]);
        if (x > bv) { bv = x; bi = g * EPC + j; }   // ids rise within a lane
      }
    }
  }
  // Row tail that does not fill a 16-byte chunk: the last chunk's workgroup.
  if (e0 + CHUNK >= V) {
    for (int v = NG * EPC + tid; v < V; v += VT) {
      const float x = DT == 1 ? __uint_as_float(
                                    (uint32_t)reinterpret_cast<const uint16_t *>(rowp)[v] << 16)
                              : reinterpret_cast<const float *>(rowp)[v];
      if (x > bv) { bv = x; bi = v; }  // (tail ids follow this lane's others)
    }
  }
  // (a lane that saw only -inf keeps key 0, below every real key)
  uint64_t key = bi == 0x7FFFFFFF ? 0ull : sel_key(bv, (uint32_t)bi);
  key = wave_max_u64(key);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = key;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = red[0];
    for (int i = 1; i < VT / kWave; ++i) m = red[i] > m ? red[i] : m;
    partials[(int64_t)r * S + s] = m;
  }
}

// One workgroup per batch row b: every (position, chunk) key is loaded by
// its own thread (one round trip) and merged into the position's maximum
// with an LDS max; then every draft is compared with its position's token at
// once, and the first mismatch ends the matches.
constexpr int kMT = 256;  // threads of the merge
__global__ __launch_bounds__(kMT) void k_verify_merge(int k, int S, const int32_t *cand,
                                                     const uint64_t *partials, int32_t *n_match,
                                                     int32_t *tokens, int32_t *next,
                                                     int32_t *k_out) {
  __shared__ unsigned long long best[kMaxVerifyK + 1];
  __shared__ int first_miss;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n = (k + 1) * S;
  const uint64_t *p = partials + (int64_t)b * n;
  for (int j = tid; j <= k; j += kMT) best[j] = 0ull;
  if (tid == 0) first_miss = k;
  __syncthreads();
  for (int i = tid; i < n; i += kMT) atomicMax(&best[i / S], (unsigned long long)p[i]);
  __syncthreads();
  auto sel = [&](int j) {  // every score -inf: the lowest id
    const uint64_t m = best[j];
    return m == 0ull ? 0 : (int)key_index(m);
  };
  for (int j = tid; j < k; j += kMT)
    if (cand[(int64_t)b * k + j] != sel(j)) atomicMin(&first_miss, j);
  __syncthreads();
  const int nm = first_miss;  // drafts before the first mismatch are accepted
  if (tid == 0) {
    n_match[b] = nm;
    next[b] = sel(nm);
    k_out[b] = nm == k ? k + 2 : (k - 1 > 1 ? k - 1 : 1);
  }
  for (int j = tid; j <= k; j += kMT) tokens[(int64_t)b * (k + 1) + j] = j <= nm ? sel(j) : -1;
}

// ---- the variant that allocates nothing -------------------------------------
// Its partial maxima and per-row counters live in this file-scope array
// instead of a caller workspace.  Every GPU the library runs on holds its own
// copy until the process ends; in host code the name stands for no device
// address, so the launches take the address hipGetSymbolAddress gives on
// each device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_at[kNoAllocDevices];  // per device id: the array's address, once set up
}  // namespace

hipError_t launch_verify_noalloc(const void *logits, int32_t dtype, int32_t B, int32_t k,
                                 int32_t V, int64_t row_bytes, int32_t chunks,
                                 const int32_t *cand, int32_t *n_match, int32_t *tokens,
                                 int32_t *next, int32_t *k_out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoAllocDevices) return hipErrorInvalidDevice;
  void *base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_at[dev]) {
      // set-up on this device (it is current): the array's address; nothing
      // in it needs to start at zero (every call writes the keys it reads)
      void *p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_at[dev] = p;
    }
    base = g_scratch_at[dev];
  }
  return launch_verify(logits, dtype, B, k, V, row_bytes, chunks, cand, n_match, tokens, next,
                       k_out, static_cast<uint64_t *>(base), s);
}

int verify_chunks(int32_t V, int32_t dtype) {
  const int chunk = VT * VCH * (dtype == 1 ? 8 : 4);
  return (V + chunk - 1) / chunk;
}

hipError_t launch_verify(const void *logits, int32_t dtype, int32_t B, int32_t k, int32_t V,
                         int64_t row_bytes, int32_t chunks, const int32_t *cand,
                         int32_t *n_match, int32_t *tokens, int32_t *next, int32_t *k_out,
                         uint64_t *partials, hipStream_t s) {
  if (B == 0) return hipSuccess;
  dim3 grid(chunks, B * (k + 1));
  if (dtype == 1)
    hipLaunchKernelGGL(k_verify_part<1>, grid, dim3(VT), 0, s, (const char *)logits, row_bytes,
                       V, chunks, partials);
  else
    hipLaunchKernelGGL(k_verify_part<0>, grid, dim3(VT), 0, s, (const char *)logits, row_bytes,
                       V, chunks, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_verify_merge, dim3(B), dim3(kMT), 0, s, k, chunks, cand,
                     (const uint64_t *)partials, n_match, tokens, next, k_out);
  return hipGetLastError();
}

}  // namespace tsel
