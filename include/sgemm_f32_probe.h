/*
 * Measurement support for libsgemm_f32 (not part of the GEMM contract).
 *
 * The source pages report their GEMM next to a measured FMA peak of the same
 * card ("100 Days of GPU, Day 44", opening paragraphs) and place kernels under
 * the roofline's flat compute ceiling ("Optimizing Matrix Multiply on CUDA,
 * Part 1", "The Roofline"). This probe measures that ceiling on MI355X for
 * the instruction families the SGEMM kernels use.
 */
#ifndef SGEMM_F32_PROBE_H
#define SGEMM_F32_PROBE_H

#include "sgemm_f32.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launch one peak-rate kernel on `stream` (a hipStream_t; NULL = null stream):
 *   kind 0  unpacked FP32 vector FMA (v_fmac_f32), 16 independent chains per lane
 *   kind 1  v_mfma_f32_32x32x2_f32, 4 independent accumulator blocks per wave
 *   kind 2  v_mfma_f32_16x16x4_f32, 8 independent accumulator blocks per wave
 *   kind 3  the kind-1 loop, bracketed by reads of the shader-clock counter
 *           (the one clock64() reads) and of the constant-rate counter
 *           (wall_clock64(), hipDeviceAttributeWallClockRate): lane 0 of
 *           workgroup w stores the shader-clock difference in out[256*w],
 *           lane 1 the constant-rate difference in out[256*w + 1], so
 *           out[256*w] / out[256*w + 1] * that rate is the clock workgroup w
 *           ran at. The pages log the clock beside their timings
 *           ("Optimizing Matrix Multiply on CUDA, Part 2", "Power
 *           Throttling"); keep iters small enough that the differences stay
 *           below 2^24 (exact in a float), e.g. iters <= 4096.
 * with `workgroups` workgroups of 256 lanes, each lane running `iters`
 * iterations. `out` is a caller-owned device buffer of workgroups*256 floats
 * that receives one value per lane (so the work cannot be optimised away).
 * On success stores the FLOP count of the launch in *flops (host memory) and
 * returns 0; the caller times the launch (e.g. with events on the stream).
 * Returns -1 bad kind, -2 bad workgroup count, -3 iters <= 0, -4 out NULL or
 * misaligned, -6 flops NULL, or a positive hipError_t from the launch. */
SGEMM_F32_API int sgemm_f32_peak_probe(int kind, int workgroups, int iters, float *out,
                                       void *stream, double *flops);

/* The current device's constant counter rate (the one wall_clock64() and
 * kind 3 above read) and its peak shader clock, both in kHz, as the HIP
 * runtime reports them. Returns 0, -1 if a pointer is NULL,
 * SGEMM_F32_ERR_DEVICE, or a positive hipError_t. */
SGEMM_F32_API int sgemm_f32_clock_rates(int *wall_khz, int *max_sclk_khz);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_F32_PROBE_H */
