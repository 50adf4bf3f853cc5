/*
 * gdr_calib.h - device ceilings for reading libgdr's kernel timings.
 *
 * Two plain kernels that measure what this MI355X actually sustains, so that
 * the roofline fractions of the gated delta rule kernels (gdr.h) can be set
 * beside measured ceilings as well as the datasheet peaks (HBM 8 TB/s,
 * dense fp16 matrix cores 2.5 PFLOP/s):
 *   - a streaming copy (each byte read once from HBM and written once), and
 *   - a loop of independent fp16 matrix-core products on register operands
 *     (v_mfma_f32_16x16x32_f16, the instruction the chunked kernels use).
 * Neither is part of the method; both live in libgdr so that the benchmark
 * times them with the same build and launch path.
 *
 * Conventions as in gdr.h: device pointers owned by the caller, nothing
 * allocated, freed or synchronised, launches enqueued on `hip_stream`
 * (NULL = default stream); errors are returned before any launch.
 */
#ifndef GDR_CALIB_H_
#define GDR_CALIB_H_

#include <stddef.h>
#include <stdint.h>

#include "gdr.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0 .. bytes) = src[0 .. bytes).  bytes must be a positive multiple of
 * 16 and both pointers 16-byte aligned (GDR_ERR_BAD_ALIGNMENT otherwise);
 * the buffers must not overlap.  Moves 2 * bytes through HBM when the
 * buffers are larger than the last-level cache. */
gdr_status gdr_calib_copy(const void* src, void* dst, size_t bytes, void* hip_stream);

/* `workgroups` workgroups of 256 threads; every wave issues `iters` rounds
 * of 8 independent 16x16x32 fp16 products with fp32 accumulation (16,384
 * FLOP each) and finally writes one float per thread to out[workgroups *
 * 256] (so that nothing is optimised away).  *flops receives the FLOPs the
 * launch executes: workgroups * 4 * iters * 8 * 16384.  workgroups and iters
 * must be positive (GDR_ERR_BAD_SHAPE). */
gdr_status gdr_calib_mfma(float* out, int64_t workgroups, int64_t iters, double* flops, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_CALIB_H_ */
