// launch_stubs.cpp -- stand-ins for the kernel launchers of libtsel.so, so
// that the host layer (tsel_api.cpp: argument checks, on-chip layout
// planning, kernel choice, workspace carving) can be built on its own with
// the address and undefined-behaviour sanitizers of the host compiler.  No
// launcher runs a kernel; each reports success.  Test infrastructure only.
#include <hip/hip_runtime.h>

#include "tsel_internal.hpp"

namespace tsel {

hipError_t launch_greedy(const SelectArgs &, size_t, hipStream_t) { return hipSuccess; }
hipError_t launch_topk(const SelectArgs &, const SelectArgs &, size_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_full(const SelectArgs &, int, size_t, hipStream_t, int) { return hipSuccess; }
hipError_t launch_res(const SelectArgs &, int, size_t, hipStream_t) { return hipSuccess; }
hipError_t launch_vres(const SelectArgs &, int, size_t, hipStream_t) { return hipSuccess; }
hipError_t launch_renorm(const SelectArgs &, size_t, float *, int64_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_logprob(const float *, int64_t, int32_t, int32_t, const int32_t *, float *,
                          hipStream_t) {
  return hipSuccess;
}
hipError_t launch_vsel_expand(const int32_t *, int32_t, const int32_t *, int32_t, int32_t,
                              const int32_t *, int32_t *, int32_t, int32_t *, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_vsel_match(const int32_t *, int32_t, int32_t, const int32_t *, int32_t *,
                             int32_t *, int32_t *, int32_t *, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_verify(const void *, int32_t, int32_t, int32_t, int32_t, int64_t, int32_t,
                         const int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, uint64_t *,
                         hipStream_t) {
  return hipSuccess;
}
hipError_t launch_verify_noalloc(const void *, int32_t, int32_t, int32_t, int32_t, int64_t,
                                 int32_t, const int32_t *, int32_t *, int32_t *, int32_t *,
                                 int32_t *, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_repack(const void *, int32_t, int64_t, void *, int64_t, int32_t, int32_t,
                         hipStream_t) {
  return hipSuccess;
}
hipError_t launch_finish(int32_t, const int32_t *, const int32_t *, const int32_t *,
                         const int32_t *, int32_t, uint8_t *, int32_t *, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_mask_build(int32_t, const int32_t *, int32_t, uint32_t *, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_beam(const BeamArgs &, hipStream_t) { return hipSuccess; }

// Sizes the kernels' own files define (the chunking of verification and the
// beam kernel's LDS), restated for the stand-in build.
int verify_chunks(int32_t V, int32_t dtype) {
  const int chunk = 256 * 8 * (dtype == 1 ? 8 : 4);
  return (V + chunk - 1) / chunk;
}
size_t beam_rows_lds(int32_t V) {
  const size_t mw = ((size_t)V + 31) / 32;
  return (((2 * mw + 3) & ~size_t(3)) + kBeamSelBins) * 4 + (size_t)kSelCap * 8;
}

}  // namespace tsel
