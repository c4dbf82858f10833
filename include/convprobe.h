/*
 * convprobe -- peak-rate probes for the roofline denominators (measurement
 * support, not part of the convolution path).  A benchmark reports the
 * rates these kernels reach beside the published MI355X figures.
 *
 * All calls enqueue one kernel on `stream` (a hipStream_t, NULL = null
 * stream), allocate nothing, do not synchronise, and return a hipError_t
 * code (0 = success; hipErrorInvalidValue for bad arguments, checked before
 * any launch).  The caller times them with events on the same stream.
 */
#ifndef CONVPROBE_H
#define CONVPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads per workgroup of every probe kernel (256). */
int32_t conv_probe_threads(void);

/* Back-to-back MFMA work: kind 0 = v_mfma_f32_32x32x16_bf16, kind 1 =
 * v_mfma_f32_16x16x4_f32, kind 2 = v_mfma_f32_16x16x32_bf16, `iters` rounds
 * of independent accumulator chains per wave, `grid` workgroups.  sink:
 * device buffer of grid * 256 floats (each lane writes its accumulator
 * sum).  *flop (may be NULL) receives the useful work the launch performs
 * (2*M*N*K per instruction).  kind 3 is an LDS read-rate probe instead
 * (16-byte conflict-free reads, eight in flight per wave); *flop then
 * receives the bytes it reads from LDS. */
int32_t conv_probe_mfma(int32_t kind, int32_t iters, int32_t grid, void *sink, void *stream, double *flop);

/* Streaming read of `bytes` (a multiple of 16, >= 16) from device buffer
 * `buf` (16-byte aligned) with `grid` workgroups; sink: device buffer of
 * grid * 256 uint32 (each lane writes the XOR of what it read). */
int32_t conv_probe_hbm_read(const void *buf, int64_t bytes, int32_t grid, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVPROBE_H */
