/*
 * tsel_probe.h -- libtsel_probe.so, diagnostics kept out of libtsel.so: the
 * HBM read rate a plain streaming kernel reaches, and a check of the device
 * exp2 instruction the sampling kernels depend on.  Neither computes any
 * part of the decode step.  Both return 0, or a HIP error code (hipError_t
 * as int); both only enqueue work on `stream` (NULL: the default stream).
 */
#ifndef TSEL_PROBE_H
#define TSEL_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * tsel_probe_read -- reads `bytes` (a multiple of 16) from the 16-byte
 * aligned device buffer `src` once, with `blocks` workgroups of 256 lanes,
 * 16-byte loads, four in flight per lane.  `out` is one device word the
 * kernel may write (to keep the loads live).  The caller times the launch;
 * bytes / time is the read rate.
 * Errors: hipErrorInvalidValue for NULL pointers, bytes % 16 != 0 or
 * blocks < 1.
 */
int tsel_probe_read(const void *src, size_t bytes, int blocks, uint32_t *out, void *stream);

/*
 * tsel_probe_exp2_monotone -- counts the binary32 inputs x in [lo, hi]
 * (numeric order, -0 and +0 one point) for which the device exp2 instruction
 * gives exp2(next(x)) < exp2(x), and adds the count to the device uint64
 * `*violations` (the caller zeroes it first).  Sampling without top_k maps
 * histogram bins of exp2 masses back to score intervals, which needs 0 here.
 * Errors: hipErrorInvalidValue for NULL violations, NaN bounds or lo > hi.
 */
int tsel_probe_exp2_monotone(float lo, float hi, unsigned long long *violations, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TSEL_PROBE_H */
