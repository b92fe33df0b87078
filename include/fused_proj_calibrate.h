/*
 * fused_proj_calibrate.h — measurement aid beside the fused projection's C ABI.
 *
 * Not part of the projection: the benchmark uses this call to put the fused kernel's
 * throughput beside the rate the matrix cores of this GPU sustain on their own. The
 * published dense bf16 peak (2.5 PFLOP/s) assumes the top clock; a stream of MFMAs on
 * varied data draws enough power that the chip lowers its clock, and this call measures
 * what remains.
 *
 * Memory: the caller owns every device buffer. Errors are the FUSED_PROJ_* codes of
 * fused_proj.h.
 */
#ifndef FUSED_PROJ_CALIBRATE_H
#define FUSED_PROJ_CALIBRATE_H

#include <stddef.h>

#include "fused_proj.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueues on `stream` (a hipStream_t; NULL = the legacy default stream) one launch of a
 * kernel that issues nothing but bf16 v_mfma_f32_32x32x16_bf16 instructions: one
 * workgroup of 4 waves (one per SIMD) per CU of the current device, each wave
 * `iterations` x 16 MFMAs on 8 independent accumulators, its operands four sets of
 * pseudo-random bf16 values in [-1, 1) derived from `seed`. The launch performs
 * *flops_per_launch = CUs * 4 * iterations * 16 * 32768 floating-point operations; time
 * it with events on the same stream. Each thread writes one float of its accumulators to
 * sink[workgroup * 256 + thread], so sink must hold CUs * 256 floats (sink_bytes).
 * Returns immediately (no synchronisation, no allocation). Errors: FUSED_PROJ_EINVAL
 * (iterations < 1, flops_per_launch or sink NULL, sink_bytes too small), FUSED_PROJ_EHIP
 * (device query or launch failure). */
int fused_proj_mfma_ceiling(int iterations, unsigned seed, float *sink, size_t sink_bytes, void *stream,
                            double *flops_per_launch);

#ifdef __cplusplus
}
#endif

#endif /* FUSED_PROJ_CALIBRATE_H */
