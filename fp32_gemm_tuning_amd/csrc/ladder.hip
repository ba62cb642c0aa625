// The pages' optimisation ladder, rebuilt for wave64 gfx950. Each rung is a
// complete, edge-guarded SGEMM (the pages' kernels assume whole tiles; these
// accept any M, N, K and leading dimensions). They exist as evidence: the
// same contract as the main kernels, timed and profiled side by side.
//
//   naive       one lane per output, lanes walk down a column of C
//               ("GEMM from scratch", Module 02)
//   coalesced   lanes walk along a row of C (Module 03; "Optimizing Matrix
//               Multiply on CUDA, Part 1", "Stage 1: Coalescing")
//   lds_tiled   16x16 tiles of A and B staged in LDS, two barriers per slice
//               (Module 04; Part 1, "Stage 2: Shared-Memory Tiling";
//               "100 Days of GPU, Day 44", step 3)
//   reg1d       64x64 block tile, each lane a column of 8 outputs
//               (Module 05, kernel 4; Day 44 step 4)
//   reg2d       128x128 block tile, each lane an 8x8 patch, outer product per
//               k (Module 05; Part 1, "Stage 3: Register Tiling"; Day 44 step 5)
//   vec4_transa reg2d plus 16-byte global loads and an A tile stored
//               transposed, with the fill that scatters each 16-byte load down
//               a column, unpadded (Module 06; Day 44 step 6)
#include "kernels.hpp"
#include "sgemm_f32.h"

namespace sgemm {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t max_workgroups(int threads) { return (int64_t)INT32_MAX / threads; }

static int check_grid(int64_t tiles, int threads) {
    return tiles <= max_workgroups(threads) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// C = beta * C
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scale(Args a) {
    const int tiles_n = (a.N + 255) / 256;
    const int64_t i = blockIdx.x / tiles_n;
    const int64_t j = (int64_t)(blockIdx.x % tiles_n) * 256 + threadIdx.x;
    if (i < a.M && j < a.N) {
        float* p = a.C + i * a.ldc + j;
        *p = (a.beta != 0.0f) ? a.beta * *p : 0.0f;
    }
}

hipError_t launch_scale(const Args& a, hipStream_t s) {
    const int64_t wgs = (int64_t)a.M * cdiv(a.N, 256);
    if (wgs > max_workgroups(256)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_scale, dim3((unsigned)wgs), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// naive: a 256-lane workgroup covers 16x16 outputs; lane l takes row l%16,
// so the 64 lanes of a wave sit on 16 different rows of A (uncoalesced).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_naive(Args a) {
    const int tiles_n = (a.N + 15) / 16;
    const int64_t i = (int64_t)(blockIdx.x / tiles_n) * 16 + (threadIdx.x & 15);
    const int64_t j = (int64_t)(blockIdx.x % tiles_n) * 16 + (threadIdx.x >> 4);
    if (i < a.M && j < a.N) {
        const float* ap = a.A + i * a.lda;
        const float* bp = a.B + j;
        float s = 0.0f;
        for (int k = 0; k < a.K; ++k) s += ap[k] * bp[(int64_t)k * a.ldb];
        store_out(a, i, j, s);
    }
}

static int check_naive(const Args& a) { return check_grid(cdiv(a.M, 16) * cdiv(a.N, 16), 256); }
static hipError_t launch_naive(const Args& a, hipStream_t s) {
    hipLaunchKernelGGL(k_naive, dim3((unsigned)(cdiv(a.M, 16) * cdiv(a.N, 16))), dim3(256), 0, s,
                       a);
    return hipGetLastError();
}
Variant kNaive = {"naive", check_naive, launch_naive, (const void*)k_naive, 256};

// ---------------------------------------------------------------------------
// coalesced: a workgroup covers 4 rows x 64 columns; each wave is one row of
// 64 consecutive outputs, so its B reads and C writes are contiguous and its
// A reads are one broadcast address.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_coalesced(Args a) {
    const int tiles_n = (a.N + 63) / 64;
    const int64_t i = (int64_t)(blockIdx.x / tiles_n) * 4 + (threadIdx.x >> 6);
    const int64_t j = (int64_t)(blockIdx.x % tiles_n) * 64 + (threadIdx.x & 63);
    if (i < a.M && j < a.N) {
        const float* ap = a.A + i * a.lda;
        const float* bp = a.B + j;
        float s = 0.0f;
        for (int k = 0; k < a.K; ++k) s += ap[k] * bp[(int64_t)k * a.ldb];
        store_out(a, i, j, s);
    }
}

static int check_coalesced(const Args& a) { return check_grid(cdiv(a.M, 4) * cdiv(a.N, 64), 256); }
static hipError_t launch_coalesced(const Args& a, hipStream_t s) {
    hipLaunchKernelGGL(k_coalesced, dim3((unsigned)(cdiv(a.M, 4) * cdiv(a.N, 64))), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}
Variant kCoalesced = {"coalesced", check_coalesced, launch_coalesced,
                            (const void*)k_coalesced, 256};

// ---------------------------------------------------------------------------
// lds_tiled: 16x16 output tile, 16-deep K slices of A and B in LDS. The first
// barrier makes the slice visible, the second keeps it alive until every
// lane has finished reading it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_lds_tiled(Args a) {
    __shared__ float As[16][16];
    __shared__ float Bs[16][16];
    const int tiles_n = (a.N + 15) / 16;
    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
    const int64_t i = (int64_t)(blockIdx.x / tiles_n) * 16 + ty;
    const int64_t j = (int64_t)(blockIdx.x % tiles_n) * 16 + tx;
    float s = 0.0f;
    for (int k0 = 0; k0 < a.K; k0 += 16) {
        As[ty][tx] = (i < a.M && k0 + tx < a.K) ? a.A[i * a.lda + k0 + tx] : 0.0f;
        Bs[ty][tx] = (k0 + ty < a.K && j < a.N) ? a.B[(int64_t)(k0 + ty) * a.ldb + j] : 0.0f;
        __syncthreads();
#pragma unroll
        for (int d = 0; d < 16; ++d) s += As[ty][d] * Bs[d][tx];
        __syncthreads();
    }
    if (i < a.M && j < a.N) store_out(a, i, j, s);
}

static int check_lds_tiled(const Args& a) { return check_grid(cdiv(a.M, 16) * cdiv(a.N, 16), 256); }
static hipError_t launch_lds_tiled(const Args& a, hipStream_t s) {
    hipLaunchKernelGGL(k_lds_tiled, dim3((unsigned)(cdiv(a.M, 16) * cdiv(a.N, 16))), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}
Variant kLdsTiled = {"lds_tiled", check_lds_tiled, launch_lds_tiled,
                           (const void*)k_lds_tiled, 256};

// ---------------------------------------------------------------------------
// reg1d: 64x64 block tile, 8-deep slices, 512 lanes; lane (ty, tx) owns rows
// 8*ty .. 8*ty+7 of column tx. One B value from LDS feeds 8 FMAs; the A values
// are the same address across a wave (broadcast).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void k_reg1d(Args a) {
    __shared__ float As[64][8];
    __shared__ float Bs[8][64];
    const int tiles_n = (a.N + 63) / 64;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * 64;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * 64;
    const int t = threadIdx.x;
    const int tx = t & 63, ty = t >> 6;
    const int ar = t >> 3, ac = t & 7;
    const int br = t >> 6, bc = t & 63;
    float acc[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
    for (int k0 = 0; k0 < a.K; k0 += 8) {
        As[ar][ac] = (m0 + ar < a.M && k0 + ac < a.K) ? a.A[(m0 + ar) * a.lda + k0 + ac] : 0.0f;
        Bs[br][bc] = (k0 + br < a.K && n0 + bc < a.N)
                         ? a.B[(int64_t)(k0 + br) * a.ldb + n0 + bc] : 0.0f;
        __syncthreads();
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const float b = Bs[d][tx];
#pragma unroll
            for (int r = 0; r < 8; ++r) acc[r] += As[ty * 8 + r][d] * b;
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int64_t i = m0 + ty * 8 + r, j = n0 + tx;
        if (i < a.M && j < a.N) store_out(a, i, j, acc[r]);
    }
}

static int check_reg1d(const Args& a) { return check_grid(cdiv(a.M, 64) * cdiv(a.N, 64), 512); }
static hipError_t launch_reg1d(const Args& a, hipStream_t s) {
    hipLaunchKernelGGL(k_reg1d, dim3((unsigned)(cdiv(a.M, 64) * cdiv(a.N, 64))), dim3(512), 0, s,
                       a);
    return hipGetLastError();
}
Variant kReg1d = {"reg1d", check_reg1d, launch_reg1d, (const void*)k_reg1d, 512};

// ---------------------------------------------------------------------------
// Shared by reg2d and vec4_transa: a 128x128 block of C cut into 256 patches
// of 8x8, one per lane (lane l: patch row l / 16, patch column l % 16), held
// in registers while 8-deep slices of A and B pass through LDS.
// ---------------------------------------------------------------------------
struct Patch {
    float v[8][8];
    __device__ void clear() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
    // One k step: the 8 A values of the patch's rows times the 8 B values of
    // its columns, 64 FMAs.
    __device__ void rank1(const float (&from_a)[8], const float (&from_b)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) v[i][j] += from_a[i] * from_b[j];
    }
    // Epilogue for the patch whose first output is (row0, col0); outputs
    // past the matrix edges are skipped.
    __device__ void store(const Args& a, int64_t row0, int64_t col0) const {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (row0 + i < a.M && col0 + j < a.N) store_out(a, row0 + i, col0 + j, v[i][j]);
    }
};

// ---------------------------------------------------------------------------
// reg2d: A's slice kept as it is stored (128 rows x 8 k), B's as 8 k x 128
// columns; the 1024 elements of each slice are loaded four per lane with
// 4-byte loads, element e of a slice at (e / width, e % width).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_reg2d(Args a) {
    __shared__ float slice_a[128][8];
    __shared__ float slice_b[8][128];
    const int cols_of_blocks = (a.N + 127) / 128;
    const int64_t bm = (int64_t)(blockIdx.x / cols_of_blocks) * 128;
    const int64_t bn = (int64_t)(blockIdx.x % cols_of_blocks) * 128;
    const int lane = threadIdx.x;
    const int pm = (lane >> 4) * 8, pn = (lane & 15) * 8;   // patch origin in the block
    Patch acc;
    acc.clear();
    for (int64_t k0 = 0; k0 < a.K; k0 += 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = q * 256 + lane;
            const int64_t am = bm + e / 8, ak = k0 + e % 8;
            slice_a[e / 8][e % 8] = (am < a.M && ak < a.K) ? a.A[am * a.lda + ak] : 0.0f;
            const int64_t bk = k0 + e / 128, bnn = bn + e % 128;
            slice_b[e / 128][e % 128] = (bk < a.K && bnn < a.N) ? a.B[bk * a.ldb + bnn] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            float from_a[8], from_b[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                from_a[u] = slice_a[pm + u][kk];
                from_b[u] = slice_b[kk][pn + u];
            }
            acc.rank1(from_a, from_b);
        }
        __syncthreads();
    }
    acc.store(a, bm + pm, bn + pn);
}

static int check_reg2d(const Args& a) { return check_grid(cdiv(a.M, 128) * cdiv(a.N, 128), 256); }
static hipError_t launch_reg2d(const Args& a, hipStream_t s) {
    hipLaunchKernelGGL(k_reg2d, dim3((unsigned)(cdiv(a.M, 128) * cdiv(a.N, 128))), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}
Variant kReg2d = {"reg2d", check_reg2d, launch_reg2d, (const void*)k_reg2d, 256};

// ---------------------------------------------------------------------------
// vec4_transa: reg2d with 16-byte global loads, and A's slice kept k-major
// (slice_at[k][m]) so that a patch's 8 A values for one k are adjacent: two
// 16-byte LDS reads, like B's. Each lane loads one 16-byte chunk of A (block
// row lane / 2, k offset 4 * (lane % 2)) and writes its four floats down
// column m of slice_at. The two lanes of a row write rows k and k + 4 of
// that column, 4 * 128 floats apart, which is the same LDS bank: a two-way
// store conflict. The rung keeps it, unpadded, as the baseline the main
// kernels remove (they never store A transposed).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_vec4_transa(Args a) {
    __shared__ __attribute__((aligned(16))) float slice_at[8][128];
    __shared__ __attribute__((aligned(16))) float slice_b[8][128];
    const int cols_of_blocks = (a.N + 127) / 128;
    const int64_t bm = (int64_t)(blockIdx.x / cols_of_blocks) * 128;
    const int64_t bn = (int64_t)(blockIdx.x % cols_of_blocks) * 128;
    const int lane = threadIdx.x;
    const int pm = (lane >> 4) * 8, pn = (lane & 15) * 8;
    const int fill_m = lane >> 1, fill_k = (lane & 1) * 4;        // A chunk of this lane
    const int fill_kb = lane >> 5, fill_n = (lane & 31) * 4;      // B chunk of this lane
    Patch acc;
    acc.clear();
    for (int64_t k0 = 0; k0 < a.K; k0 += 8) {
        // K and N are multiples of 4 (checked on the host), so a chunk lies
        // wholly inside the matrix or wholly outside it.
        f32x4 ca = {0.0f, 0.0f, 0.0f, 0.0f}, cb = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bm + fill_m < a.M && k0 + fill_k < a.K)
            ca = *(const f32x4*)(a.A + (bm + fill_m) * a.lda + k0 + fill_k);
        if (k0 + fill_kb < a.K && bn + fill_n < a.N)
            cb = *(const f32x4*)(a.B + (k0 + fill_kb) * a.ldb + bn + fill_n);
#pragma unroll
        for (int c = 0; c < 4; ++c) slice_at[fill_k + c][fill_m] = ca[c];
        *(f32x4*)&slice_b[fill_kb][fill_n] = cb;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            float from_a[8], from_b[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 va = *(const f32x4*)&slice_at[kk][pm + 4 * h];
                const f32x4 vb = *(const f32x4*)&slice_b[kk][pn + 4 * h];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    from_a[4 * h + c] = va[c];
                    from_b[4 * h + c] = vb[c];
                }
            }
            acc.rank1(from_a, from_b);
        }
        __syncthreads();
    }
    acc.store(a, bm + pm, bn + pn);
}

static int check_vec4_transa(const Args& a) {
    if ((a.K & 3) || (a.N & 3) || (a.lda & 3) || (a.ldb & 3) || !aligned16(a.A) ||
        !aligned16(a.B))
        return SGEMM_F32_ERR_UNSUPPORTED;
    return check_grid(cdiv(a.M, 128) * cdiv(a.N, 128), 256);
}
static hipError_t launch_vec4_transa(const Args& a, hipStream_t s) {
    hipLaunchKernelGGL(k_vec4_transa, dim3((unsigned)(cdiv(a.M, 128) * cdiv(a.N, 128))),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}
Variant kVec4TransA = {"vec4_transa", check_vec4_transa, launch_vec4_transa,
                             (const void*)k_vec4_transa, 256};

}  // namespace sgemm
