// Peak-rate microbenchmarks: how many FP32 FLOP/s the chip sustains for the
// two instruction families the SGEMM kernels use, measured rather than
// assumed (the pages measure an FMA peak next to their GEMM for the same
// reason: "100 Days of GPU, Day 44", opening paragraphs, and the roofline's
// flat ceiling in "Optimizing Matrix Multiply on CUDA, Part 1", "The
// Roofline").
//
//   kind 0: unpacked v_fmac_f32 (VOP2, all operands in VGPRs, the form the
//           vector GEMM kernels' inner loops compile to), 16 independent
//           accumulators per lane
//   kind 1: v_mfma_f32_32x32x2_f32, 4 independent accumulators per wave
//   kind 2: v_mfma_f32_16x16x4_f32, 8 independent accumulators per wave
//   kind 3: the kind-1 loop between two reads of the shader-clock counter
//           and of the constant-rate counter; lane 0 of each workgroup
//           stores both differences, whose ratio times the constant rate
//           is the clock the matrix cores ran at (the pages log the clock
//           next to their timings: "Optimizing Matrix Multiply on CUDA,
//           Part 2", "Power Throttling")
// Each lane writes one float derived from all its chains, so nothing is
// dead code; the values stay small and normal.
#include "kernels.hpp"
#include "sgemm_f32_probe.h"

namespace sgemm {

constexpr int PK_THREADS = 256;

__global__ __launch_bounds__(PK_THREADS) void k_peak_fma(float* out, int iters, float x) {
    float acc[16], m[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        acc[j] = 0.0f;
        m[j] = 1e-3f * x * (float)(threadIdx.x + j);
    }
    const float b = 1e-4f * x * (float)(threadIdx.x & 7);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = __builtin_fmaf(m[j], b, acc[j]);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[j];
    out[blockIdx.x * PK_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PK_THREADS) void k_peak_mfma32(float* out, int iters, float x) {
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    const float a = 1e-3f * x * (float)(threadIdx.x & 63);
    const float b = 1e-4f * x;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[blockIdx.x * PK_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PK_THREADS) void k_peak_mfma16(float* out, int iters, float x) {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float a = 1e-3f * x * (float)(threadIdx.x & 63);
    const float b = 1e-4f * x;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[blockIdx.x * PK_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(PK_THREADS) void k_clock_mfma32(float* out, int iters, float x) {
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    const float a = 1e-3f * x * (float)(threadIdx.x & 63);
    const float b = 1e-4f * x;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    // The sum depends on every MFMA, so the second reads come after them.
    __builtin_amdgcn_s_waitcnt(0);
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float v = s;
    if (threadIdx.x == 0) v = (float)(c1 - c0);
    if (threadIdx.x == 1) v = (float)(r1 - r0);
    out[blockIdx.x * PK_THREADS + threadIdx.x] = v;
}

}  // namespace sgemm

using namespace sgemm;

extern "C" SGEMM_F32_API int sgemm_f32_peak_probe(int kind, int workgroups, int iters, float* out,
                                                  void* stream, double* flops) {
    if (kind < 0 || kind > 3) return -1;
    if (workgroups <= 0 || (int64_t)workgroups > max_workgroups(PK_THREADS)) return -2;
    if (iters <= 0) return -3;
    if (out == nullptr || (reinterpret_cast<uintptr_t>(out) & 3u)) return -4;
    if (flops == nullptr) return -6;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const double lanes = (double)workgroups * PK_THREADS;
    const double waves = lanes / 64.0;
    switch (kind) {
        case 0:
            hipLaunchKernelGGL(k_peak_fma, dim3(workgroups), dim3(PK_THREADS), 0, s, out, iters, 1.0f);
            *flops = lanes * iters * 16.0 * 2.0;
            break;
        case 1:
            hipLaunchKernelGGL(k_peak_mfma32, dim3(workgroups), dim3(PK_THREADS), 0, s, out, iters,
                               1.0f);
            *flops = waves * iters * 4.0 * (2.0 * 32 * 32 * 2);
            break;
        case 2:
            hipLaunchKernelGGL(k_peak_mfma16, dim3(workgroups), dim3(PK_THREADS), 0, s, out, iters,
                               1.0f);
            *flops = waves * iters * 8.0 * (2.0 * 16 * 16 * 4);
            break;
        default:
            hipLaunchKernelGGL(k_clock_mfma32, dim3(workgroups), dim3(PK_THREADS), 0, s, out,
                               iters, 1.0f);
            *flops = waves * iters * 4.0 * (2.0 * 32 * 32 * 2);
            break;
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

extern "C" SGEMM_F32_API int sgemm_f32_clock_rates(int* wall_khz, int* max_sclk_khz) {
    if (wall_khz == nullptr || max_sclk_khz == nullptr) return -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SGEMM_F32_ERR_DEVICE;
    hipError_t e = hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return (int)e;
    e = hipDeviceGetAttribute(max_sclk_khz, hipDeviceAttributeClockRate, dev);
    return e == hipSuccess ? 0 : (int)e;
}
