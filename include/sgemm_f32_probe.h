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
 * with `workgroups` workgroups of 256 lanes, each lane running `iters`
 * iterations. `out` is a caller-owned device buffer of workgroups*256 floats
 * that receives one value per lane (so the work cannot be optimised away).
 * On success stores the FLOP count of the launch in *flops (host memory) and
 * returns 0; the caller times the launch (e.g. with events on the stream).
 * Returns -1 bad kind, -2 bad workgroup count, -3 iters <= 0, -4 out NULL or
 * misaligned, -6 flops NULL, or a positive hipError_t from the launch. */
SGEMM_F32_API int sgemm_f32_peak_probe(int kind, int workgroups, int iters, float *out,
                                       void *stream, double *flops);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_F32_PROBE_H */
