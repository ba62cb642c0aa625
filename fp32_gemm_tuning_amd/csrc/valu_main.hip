// Vector-FMA main kernel (no matrix cores): the end point of the pages' CUDA
// ladder, re-planned for wave64 gfx950.
//
//  - 128x128 block tile, 16-deep K slices (BK 32 -> 16 halves the transposed
//    fill's store passes: "Optimizing Matrix Multiply on CUDA, Part 2",
//    "Reducing the Slice Depth"), 256 lanes.
//  - Warp tiling for wave64: each wave owns a compact 64x64 sub-tile, an 8x8
//    grid of lanes ("Part 2", "Assigning a Compact Tile to Each Warp").
//  - Each lane's 8x8 patch is split into two groups of 4 rows and 4 columns
//    32 apart ("Part 2", "Changing the Shared-Memory Access Pattern"), so
//    the 8 lanes that share a row of the wave's lane grid read 8 consecutive
//    16-byte B chunks and 8 lanes that share a column read one broadcast A
//    chunk: no LDS read conflicts.
//  - A is stored transposed (As[k][m]) so a lane's 4+4 A values are two
//    16-byte LDS loads ("GEMM from scratch", Module 06). The fill assigns
//    consecutive lanes to consecutive rows m of A, so each scattered 4-byte
//    store of a 16-byte global load writes 64 consecutive floats of one As
//    row: no store conflicts either, with no padding (the pages' fill put
//    two lanes 512 floats apart in one bank: "100 Days of GPU, Day 44",
//    "Two ladders, one kernel").
//  - Double-buffered K loop with a register prefetch stage and one barrier
//    per slice ("Part 2", "Overlapping Loads and Computation").
//  - Plain (unpacked) v_fmac_f32: packed FP32 FMA is disabled at build time.
//    Unpacked FMAs still run above half the chip's 157.3 TFLOP/s vector
//    peak (the peak probe and this kernel both exceed 78.6), so the kernel
//    is priced against the full vector peak.
#include "kernels.hpp"
#include "sgemm_f32.h"

namespace sgemm {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int V_BM = 128, V_BN = 128, V_BK = 16, V_NT = 256, V_GROUP_M = 8;

template <bool VEC>
struct ValuFill {
    static constexpr int AE = V_BM * V_BK / V_NT;  // 8 floats of A per lane per slice
    static constexpr int BE = V_BK * V_BN / V_NT;  // 8 floats of B
    f32x4 ra[AE / 4];
    f32x4 rb[BE / 4];

    __device__ __forceinline__ void load(const Args& a, int t, int m0, int n0, int k0,
                                         int rows_valid, int cols_valid) {
        const int kk = (a.K - k0) < V_BK ? (a.K - k0) : V_BK;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(
            a.A + (int64_t)m0 * a.lda + k0, (uint32_t)(((int64_t)(rows_valid - 1) * a.lda + kk) * 4));
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(
            a.B + (int64_t)k0 * a.ldb + n0, (uint32_t)(((int64_t)(kk - 1) * a.ldb + cols_valid) * 4));
        if (VEC) {
#pragma unroll
            for (int p = 0; p < AE / 4; ++p) {
                const int c = t + V_NT * p, m = c & (V_BM - 1), q = c >> 7;
                const bool ok = m < rows_valid && 4 * q + 4 <= kk;
                ra[p] = buf_load4(rA, ok ? (uint32_t)((m * (int)a.lda + 4 * q) * 4) : OOB);
            }
#pragma unroll
            for (int p = 0; p < BE / 4; ++p) {
                const int c = t + V_NT * p, krow = c >> 5, nq = c & 31;
                const bool ok = krow < kk && 4 * nq + 4 <= cols_valid;
                rb[p] = buf_load4(rB, ok ? (uint32_t)((krow * (int)a.ldb + 4 * nq) * 4) : OOB);
            }
        } else {
#pragma unroll
            for (int p = 0; p < AE; ++p) {
                const int e = t + V_NT * p, m = e & (V_BM - 1), kq = e >> 7;
                const bool ok = m < rows_valid && kq < kk;
                ra[p >> 2][p & 3] = buf_load1(rA, ok ? (uint32_t)((m * (int)a.lda + kq) * 4) : OOB);
            }
#pragma unroll
            for (int p = 0; p < BE; ++p) {
                const int e = t + V_NT * p, krow = e >> 7, n = e & (V_BN - 1);
                const bool ok = krow < kk && n < cols_valid;
                rb[p >> 2][p & 3] = buf_load1(rB, ok ? (uint32_t)((krow * (int)a.ldb + n) * 4) : OOB);
            }
        }
    }

    // As[k][m] (pitch V_BM), Bs[k][n] (pitch V_BN).
    __device__ __forceinline__ void store(float* As, float* Bs, int t) const {
        if (VEC) {
#pragma unroll
            for (int p = 0; p < AE / 4; ++p) {
                const int c = t + V_NT * p, m = c & (V_BM - 1), q = c >> 7;
#pragma unroll
                for (int e = 0; e < 4; ++e) As[(4 * q + e) * V_BM + m] = ra[p][e];
            }
#pragma unroll
            for (int p = 0; p < BE / 4; ++p) {
                const int c = t + V_NT * p, krow = c >> 5, nq = c & 31;
                *(f32x4*)&Bs[krow * V_BN + 4 * nq] = rb[p];
            }
        } else {
#pragma unroll
            for (int p = 0; p < AE; ++p) {
                const int e = t + V_NT * p, m = e & (V_BM - 1), kq = e >> 7;
                As[kq * V_BM + m] = ra[p >> 2][p & 3];
            }
#pragma unroll
            for (int p = 0; p < BE; ++p) {
                const int e = t + V_NT * p, krow = e >> 7, n = e & (V_BN - 1);
                Bs[krow * V_BN + n] = rb[p >> 2][p & 3];
            }
        }
    }
};

template <bool VEC>
__global__ __launch_bounds__(256) void k_valu_main(Args a, int tiles_m, int tiles_n, int xcd_remap) {
    __shared__ __attribute__((aligned(16))) float As[2][V_BK * V_BM];
    __shared__ __attribute__((aligned(16))) float Bs[2][V_BK * V_BN];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, V_GROUP_M, xcd_remap != 0, tm, tn);
    const int m0 = tm * V_BM, n0 = tn * V_BN;
    const int rows_valid = (a.M - m0) < V_BM ? (a.M - m0) : V_BM;
    const int cols_valid = (a.N - n0) < V_BN ? (a.N - n0) : V_BN;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int ty = lane >> 3, tx = lane & 7;
    const int arow = wm * 64 + ty * 4;  // + {0..3} and + 32 + {0..3}
    const int bcol = wn * 64 + tx * 4;

    float acc[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = 0.0f;

    const int nslices = (a.K + V_BK - 1) / V_BK;
    ValuFill<VEC> fill;
    fill.load(a, t, m0, n0, 0, rows_valid, cols_valid);
    fill.store(As[0], Bs[0], t);
    __syncthreads();

    for (int s = 0; s < nslices; ++s) {
        const int cur = s & 1;
        if (s + 1 < nslices) fill.load(a, t, m0, n0, (s + 1) * V_BK, rows_valid, cols_valid);
        const float* Ac = As[cur];
        const float* Bc = Bs[cur];
        // Partial unroll: a full unroll lets the scheduler hoist all 16 steps'
        // LDS loads (256 registers of fragments) and drop to one wave per SIMD.
#pragma unroll 4
        for (int k = 0; k < V_BK; ++k) {
            const f32x4 a0 = *(const f32x4*)&Ac[k * V_BM + arow];
            const f32x4 a1 = *(const f32x4*)&Ac[k * V_BM + arow + 32];
            const f32x4 b0 = *(const f32x4*)&Bc[k * V_BN + bcol];
            const f32x4 b1 = *(const f32x4*)&Bc[k * V_BN + bcol + 32];
            const float rm[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float rn[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[r][c] += rm[r] * rn[c];
        }
        if (s + 1 < nslices) fill.store(As[cur ^ 1], Bs[cur ^ 1], t);
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int i = arow + (r & 3) + (r >> 2) * 32;
            const int j = bcol + (c & 3) + (c >> 2) * 32;
            if (i < rows_valid && j < cols_valid)
                store_out(a, (int64_t)m0 + i, (int64_t)n0 + j, acc[r][c]);
        }
}

static int check_valu_main(const Args& a) {
    const int64_t ea = ((int64_t)(V_BM - 1) * a.lda + V_BK) * 4;
    const int64_t eb = ((int64_t)(V_BK - 1) * a.ldb + V_BN) * 4;
    if (ea >= (int64_t)OOB || eb >= (int64_t)OOB) return SGEMM_F32_ERR_TOO_LARGE;
    const int64_t tiles = cdiv(a.M, V_BM) * cdiv(a.N, V_BN);
    return tiles <= max_workgroups(V_NT) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
}

static hipError_t launch_valu_main(const Args& a, hipStream_t s) {
    const int tm = (int)cdiv(a.M, V_BM), tn = (int)cdiv(a.N, V_BN);
    const dim3 grid((unsigned)((int64_t)tm * tn)), block(V_NT);
    const bool vec = !((a.K & 3) || (a.N & 3) || (a.lda & 3) || (a.ldb & 3) || !aligned16(a.A) ||
                       !aligned16(a.B));
    const int remap = xcd_remap_enabled();
    if (vec)
        hipLaunchKernelGGL(k_valu_main<true>, grid, block, 0, s, a, tm, tn, remap);
    else
        hipLaunchKernelGGL(k_valu_main<false>, grid, block, 0, s, a, tm, tn, remap);
    return hipGetLastError();
}

Variant kValuMain = {"valu_main", check_valu_main, launch_valu_main,
                           (const void*)k_valu_main<true>, V_NT};

}  // namespace sgemm
