/*
 * peak.h -- calibration kernels (libpeak.so) that measure the ceilings one MI355X
 * sustains, for reading the attention kernels' rates against a measured peak as well
 * as the published one (2.5 PFLOP/s dense bf16, 8 TB/s HBM3E).  Not part of the
 * attention path; bench.py uses them.
 *
 * All pointers are device pointers owned by the caller; `stream` is a hipStream_t (NULL:
 * the default stream).  The calls only enqueue work.  Return 0 on success, -1 for a bad
 * argument (nothing enqueued), -4 when the launch fails.
 */
#ifndef PEAK_H
#define PEAK_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Flops one peak_mfma_bf16(blocks, iters) call performs: every wave of the 256-thread
 * blocks runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16. */
double peak_mfma_bf16_flops(int blocks, int iters);

/* The MFMA loop; out: one f32 word the kernel writes only if a never-true check holds. */
int peak_mfma_bf16(int blocks, int iters, float *out, void *stream);

/* Reads `bytes` (a multiple of 16, 16-byte aligned) of buf once with 16-byte loads;
 * out: one word written only if a never-true check holds. */
int peak_stream_read(const void *buf, size_t bytes, unsigned *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PEAK_H */
