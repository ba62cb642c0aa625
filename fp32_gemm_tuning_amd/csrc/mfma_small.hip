// FP32 matrix-core kernels for shapes the tiled kernels serve badly:
// mfma_64x64_k4 (in-workgroup K split), mfma_direct (small products and few
// tiles, no LDS tile) and mfma_skinny (M <= 32, HBM-bound).
// Operand layouts and edge handling: mfma_common.hpp.
#include "mfma_common.hpp"

namespace sgemm {

// ===========================================================================
// mfma_64x64_k4: a 64x64 tile whose 4 waves split every 64-deep K slice four
// ways. Wave w multiplies k = 16w .. 16w+15 of each slice into its own full
// 64x64 accumulator (2x2 blocks of v_mfma_f32_32x32x2_f32), so each wave
// issues 32 MFMAs (2048 matrix-core cycles) per barrier -- four times the
// work of mfma_64x64 -- which hides fill latency with only one or two
// workgroups per compute unit. This is the pages' split-K idea ("Optimizing
// Matrix Multiply on CUDA, Part 2", "Selecting Among Three Kernels") moved
// inside the workgroup: the four partial tiles are summed through LDS in a
// fixed order (w = 0, 1, 2, 3), so no global workspace is needed and the
// result is deterministic.
// ===========================================================================
constexpr int KS_BM = 64, KS_BN = 64, KS_WAVES = 4, KS_BK = 16 * KS_WAVES, KS_GROUP_M = 8;

template <bool VEC>
__global__ __launch_bounds__(256) void k_mfma_ksplit(Args a, int tiles_m, int tiles_n,
                                                     int xcd_remap) {
    constexpr int BM = KS_BM, BN = KS_BN, BK = KS_BK;
    using Fill = TileFill<BM, BN, BK, 256, VEC>;
    constexpr int BNP = Fill::BNP;
    constexpr int STAGE = BM * BK + BK * BNP;  // floats per LDS stage
    static_assert(2 * STAGE >= KS_WAVES * 4 * 16 * 64, "reduction buffer must fit in the stages");
    __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, KS_GROUP_M, xcd_remap != 0, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_valid = (a.M - m0) < BM ? (a.M - m0) : BM;
    const int cols_valid = (a.N - n0) < BN ? (a.N - n0) : BN;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int h = lane >> 5, c = lane & 31;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Wave w, half h: k = 16w + 8h + s (s = 0..7) of each slice.
    const int kb = 16 * w + 8 * h;
    int aoff[2][2], boff[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
        const int row = bi * 32 + c;
#pragma unroll
        for (int v = 0; v < 2; ++v) aoff[bi][v] = row * BK + (((kb / 4 + v) ^ swz_chunk<BK>(row)) << 2);
    }
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) boff[bj] = kb * BNP + bj * 32 + c;

    const int nslices = (a.K + BK - 1) / BK;
    Fill fill;
    fill.load(a, t, m0, n0, 0, rows_valid, cols_valid);
    fill.store(smem, smem + BM * BK, t);
    __syncthreads();

    for (int s = 0; s < nslices; ++s) {
        const int cur = s & 1;
        if (s + 1 < nslices) fill.load(a, t, m0, n0, (s + 1) * BK, rows_valid, cols_valid);
        const float* Ac = smem + cur * STAGE;
        const float* Bc = Ac + BM * BK;
        float af[2][8], bf[2][8];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
            const f32x4 lo = *(const f32x4*)&Ac[aoff[bi][0]];
            const f32x4 hi = *(const f32x4*)&Ac[aoff[bi][1]];
            af[bi][0] = lo.x; af[bi][1] = lo.y; af[bi][2] = lo.z; af[bi][3] = lo.w;
            af[bi][4] = hi.x; af[bi][5] = hi.y; af[bi][6] = hi.z; af[bi][7] = hi.w;
        }
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int k = 0; k < 8; ++k) bf[bj][k] = Bc[boff[bj] + k * BNP];
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 2; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[bi][k], bf[bj][k],
                                                                       acc[bi][bj], 0, 0, 0);
        if (s + 1 < nslices) {
            float* An = smem + (cur ^ 1) * STAGE;
            fill.store(An, An + BM * BK, t);
        }
        __syncthreads();
    }

    // Fixed-order reduction: every wave parks its 4 blocks in LDS as
    // red[w][block][r][lane]; wave w then sums block w over the 4 waves.
    float* red = smem;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                red[((w * 4 + bi * 2 + bj) * 16 + r) * 64 + lane] = acc[bi][bj][r];
    __syncthreads();
    const int bi = w >> 1, bj = w & 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float v = red[((0 * 4 + w) * 16 + r) * 64 + lane];
#pragma unroll
        for (int ww = 1; ww < KS_WAVES; ++ww) v += red[((ww * 4 + w) * 16 + r) * 64 + lane];
        const int i = bi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int j = bj * 32 + c;
        if (i < rows_valid && j < cols_valid) store_out(a, (int64_t)m0 + i, (int64_t)n0 + j, v);
    }
}

static int check_ksplit(const Args& a) {
    if (!extents_ok(a, KS_BM, KS_BN, KS_BK)) return SGEMM_F32_ERR_TOO_LARGE;
    const int64_t tiles = cdiv(a.M, KS_BM) * cdiv(a.N, KS_BN);
    return tiles <= max_workgroups(256) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
}

static hipError_t launch_ksplit(const Args& a, hipStream_t s) {
    const int tm = (int)cdiv(a.M, KS_BM), tn = (int)cdiv(a.N, KS_BN);
    const dim3 grid((unsigned)((int64_t)tm * tn)), block(256);
    if (vec_ok(a))
        hipLaunchKernelGGL(k_mfma_ksplit<true>, grid, block, 0, s, a, tm, tn, xcd_remap_enabled());
    else
        hipLaunchKernelGGL(k_mfma_ksplit<false>, grid, block, 0, s, a, tm, tn, xcd_remap_enabled());
    return hipGetLastError();
}

Variant kMfmaKsplit = {"mfma_64x64_k4", check_ksplit, launch_ksplit,
                       (const void*)k_mfma_ksplit<true>, 256};

// ===========================================================================
// mfma_direct: small and medium shapes. A workgroup of KS waves owns a TM x TN
// tile of C; wave w takes the 16-deep k steps w, w + KS, w + 2*KS, ... and
// accumulates the whole tile for them (TM/32 x TN/32 blocks of
// v_mfma_f32_32x32x2_f32). Operands go straight from global memory (L2) into
// MFMA registers -- there is no LDS tile and no barrier inside the K loop, so
// the waves run independently and hide latency with a register double buffer
// (step j+KS is loaded while step j is multiplied). With the k-permuted
// operand layout a lane's A values are 8 consecutive floats of one row and its
// B values are rows of 32 consecutive columns across the half-wave. At the end
// the KS partial tiles are summed through LDS in the fixed order w = 0..KS-1.
// Fine tiles (32x32) spread a few-tile shape evenly over the compute
// units; this is the pages' split-K ("Optimizing Matrix Multiply on CUDA,
// Part 2", "Selecting Among Three Kernels") kept inside the workgroup.
// KS = 8: each wave's chain of dependent loads is half as long as with 4
// (256^3 8.8 -> 8.1 us per launch, 256x256x1000 -21%); 16 only pays at long K
// and costs at short K (64^3 +14%).
// ===========================================================================
#ifndef SGEMM_DIRECT_TM
#define SGEMM_DIRECT_TM 32
#endif
#ifndef SGEMM_DIRECT_TN
#define SGEMM_DIRECT_TN 32
#endif
#ifndef SGEMM_DIRECT_KS
#define SGEMM_DIRECT_KS 8
#endif
constexpr int DR_TM = SGEMM_DIRECT_TM, DR_TN = SGEMM_DIRECT_TN, DR_KS = SGEMM_DIRECT_KS;
constexpr int DR_GROUP_M = 8;

template <int TM, int TN, bool VEC, bool TA, bool TB>
struct DirectFrag {
    static constexpr int BI = TM / 32, BJ = TN / 32;
    float a[BI][8];
    float b[BJ][8];

    // Step starting at k0: lane (h, c) reads A[m0 + 32*bi + c][k0 + 8h + 0..7]
    // and B[k0 + 8h + s][n0 + 32*bj + c]; everything outside the matrix reads 0.
    // Element (m, k) of A sits at m*lda + k, or at k*lda + m when A is stored
    // transposed (TA); element (k, n) of B at k*ldb + n, or at n*ldb + k (TB).
    // VEC: the k-contiguous operands (A unless TA, B if TB) take 16-byte loads.
    // A step at or past the end of K (kk = 0) has empty resources: every
    // load reads zero and nothing is fetched. k0 and kk are wave-uniform;
    // readfirstlane keeps the resources in scalar registers (built from
    // vector registers, each load would run in a per-lane loop).
    __device__ __forceinline__ void load(const Args& a_, int m0, int n0, int k0_, int rows_valid,
                                         int cols_valid, int h, int c) {
        const int k0 = __builtin_amdgcn_readfirstlane(k0_);
        const int kr = a_.K - k0;
        const int kk = __builtin_amdgcn_readfirstlane(kr <= 0 ? 0 : (kr < 16 ? kr : 16));
        const __amdgpu_buffer_rsrc_t rA =
            TA ? make_rsrc(a_.A + (int64_t)k0 * a_.lda + m0,
                           kk > 0 ? (uint32_t)(((int64_t)(kk - 1) * a_.lda + rows_valid) * 4) : 0u)
               : make_rsrc(a_.A + (int64_t)m0 * a_.lda + k0,
                           kk > 0 ? (uint32_t)(((int64_t)(rows_valid - 1) * a_.lda + kk) * 4) : 0u);
        const __amdgpu_buffer_rsrc_t rB =
            TB ? make_rsrc(a_.B + (int64_t)n0 * a_.ldb + k0,
                           kk > 0 ? (uint32_t)(((int64_t)(cols_valid - 1) * a_.ldb + kk) * 4) : 0u)
               : make_rsrc(a_.B + (int64_t)k0 * a_.ldb + n0,
                           kk > 0 ? (uint32_t)(((int64_t)(kk - 1) * a_.ldb + cols_valid) * 4) : 0u);
#pragma unroll
        for (int bi = 0; bi < BI; ++bi) {
            const int row = 32 * bi + c;
            const bool rok = row < rows_valid;
            if (VEC && !TA) {
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const int kq = 8 * h + 4 * v;
                    const f32x4 x = buf_load4(rA, rok && kq + 4 <= kk ? (uint32_t)((row * (int)a_.lda + kq) * 4) : OOB);
                    a[bi][4 * v + 0] = x.x; a[bi][4 * v + 1] = x.y;
                    a[bi][4 * v + 2] = x.z; a[bi][4 * v + 3] = x.w;
                }
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int kq = 8 * h + s;
                    const int off = TA ? kq * (int)a_.lda + row : row * (int)a_.lda + kq;
                    a[bi][s] = buf_load1(rA, rok && kq < kk ? (uint32_t)(off * 4) : OOB);
                }
            }
        }
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj) {
            const int col = 32 * bj + c;
            const bool cok = col < cols_valid;
            if (VEC && TB) {
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const int kq = 8 * h + 4 * v;
                    const f32x4 x = buf_load4(rB, cok && kq + 4 <= kk ? (uint32_t)((col * (int)a_.ldb + kq) * 4) : OOB);
                    b[bj][4 * v + 0] = x.x; b[bj][4 * v + 1] = x.y;
                    b[bj][4 * v + 2] = x.z; b[bj][4 * v + 3] = x.w;
                }
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int kr = 8 * h + s;
                    const int off = TB ? col * (int)a_.ldb + kr : kr * (int)a_.ldb + col;
                    b[bj][s] = buf_load1(rB, cok && kr < kk ? (uint32_t)(off * 4) : OOB);
                }
            }
        }
    }
};

template <int TM, int TN, int KS, bool VEC, bool TA = false, bool TB = false>
__global__ __launch_bounds__(64 * KS) void k_mfma_direct(Args a, int tiles_m, int tiles_n,
                                                         int xcd_remap) {
    constexpr int BI = TM / 32, BJ = TN / 32, NB = BI * BJ;
    __shared__ float red[KS * NB * 16 * 64];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, DR_GROUP_M, xcd_remap != 0, tm, tn);
    // Workgroup- and wave-uniform values in scalar registers (the tile
    // mapping's divisions and the thread index leave them in vector ones).
    const int m0 = __builtin_amdgcn_readfirstlane(tm * TM), n0 = __builtin_amdgcn_readfirstlane(tn * TN);
    const int rows_valid = (a.M - m0) < TM ? (a.M - m0) : TM;
    const int cols_valid = (a.N - n0) < TN ? (a.N - n0) : TN;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int h = lane >> 5, c = lane & 31;

    f32x16 acc[BI][BJ];
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nsteps = (a.K + 15) / 16;
    using Frag = DirectFrag<TM, TN, VEC, TA, TB>;
    auto mma = [&](const Frag& f) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[bi][s], f.b[bj][s],
                                                                       acc[bi][bj], 0, 0, 0);
    };
    // Steps j and j + KS alternate between two register sets. The loads are
    // unconditional (past the end of K they read zeros) and fenced ahead of
    // the other set's MFMAs: loads issued on only some paths, or sunk below
    // the MFMAs, make the compiler wait for every load in flight before a
    // step's MFMAs.
    Frag f0, f1;
    f0.load(a, m0, n0, 16 * w, rows_valid, cols_valid, h, c);
    for (int j = w; j < nsteps; j += 2 * KS) {
        f1.load(a, m0, n0, 16 * (j + KS), rows_valid, cols_valid, h, c);
        __builtin_amdgcn_sched_barrier(0);
        mma(f0);
        __builtin_amdgcn_sched_barrier(0);
        f0.load(a, m0, n0, 16 * (j + 2 * KS), rows_valid, cols_valid, h, c);
        __builtin_amdgcn_sched_barrier(0);
        if (j + KS < nsteps) mma(f1);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Fixed-order reduction over the KS waves: red[w][block][r][lane].
#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                red[((w * NB + bi * BJ + bj) * 16 + r) * 64 + lane] = acc[bi][bj][r];
    __syncthreads();
    // The NB * 16 accumulators of a lane are shared out among the waves
    // (item it to wave it mod KS), each summed over the waves in order.
    for (int it = w; it < NB * 16; it += KS) {
        const int blk = it >> 4, r = it & 15;
        const int bi = blk / BJ, bj = blk % BJ;
        float v = red[((0 * NB + blk) * 16 + r) * 64 + lane];
#pragma unroll
        for (int ww = 1; ww < KS; ++ww) v += red[((ww * NB + blk) * 16 + r) * 64 + lane];
        const int i = bi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int jj = bj * 32 + c;
        if (i < rows_valid && jj < cols_valid)
            store_out(a, (int64_t)m0 + i, (int64_t)n0 + jj, v);
    }
}

// The 16-byte loads need every k-contiguous operand (A unless transposed, B
// if transposed) 16-byte aligned with a row pitch and K that are multiples of 4.
static bool small_vec_ok(const Args& a) {
    if (a.K & 3) return false;
    if (!a.ta && ((a.lda & 3) || !aligned16(a.A))) return false;
    if (a.tb && ((a.ldb & 3) || !aligned16(a.B))) return false;
    return true;
}

// Largest byte extent one buffer resource of an operand spans: `rows` x
// `depth` of A (M rows by K) or B (K by N columns) in its storage order.
static int64_t extent_a(const Args& a, int rows, int depth) {
    return (a.ta ? (int64_t)(depth - 1) * a.lda + rows : (int64_t)(rows - 1) * a.lda + depth) * 4;
}
static int64_t extent_b(const Args& a, int depth, int cols) {
    return (a.tb ? (int64_t)(cols - 1) * a.ldb + depth : (int64_t)(depth - 1) * a.ldb + cols) * 4;
}

static int check_direct(const Args& a) {
    const int64_t ea = extent_a(a, DR_TM, 16);
    const int64_t eb = extent_b(a, 16, DR_TN);
    if (ea >= (int64_t)OOB || eb >= (int64_t)OOB) return SGEMM_F32_ERR_TOO_LARGE;
    const int64_t tiles = cdiv(a.M, DR_TM) * cdiv(a.N, DR_TN);
    return tiles <= max_workgroups(64 * DR_KS) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
}

static hipError_t launch_direct(const Args& a, hipStream_t s) {
    const int tm = (int)cdiv(a.M, DR_TM), tn = (int)cdiv(a.N, DR_TN);
    const dim3 grid((unsigned)((int64_t)tm * tn)), block(64 * DR_KS);
    const bool vec = small_vec_ok(a);
    return with_trans(a, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        if (vec)
            hipLaunchKernelGGL((k_mfma_direct<DR_TM, DR_TN, DR_KS, true, TA, TB>), grid, block, 0, s,
                               a, tm, tn, xcd_remap_enabled());
        else
            hipLaunchKernelGGL((k_mfma_direct<DR_TM, DR_TN, DR_KS, false, TA, TB>), grid, block, 0, s,
                               a, tm, tn, xcd_remap_enabled());
        return hipGetLastError();
    });
}

Variant kMfmaDirect = {"mfma_direct", check_direct, launch_direct,
                       (const void*)k_mfma_direct<DR_TM, DR_TN, DR_KS, true>, 64 * DR_KS, true,
                       nullptr, nullptr, DR_TM, DR_TN, 16};

// ===========================================================================
// mfma_skinny: for few rows (near-GEMV, e.g. 16 x 8192 x 8192, where B is
// read once and the shape is bound by HBM bandwidth). A workgroup owns a
// 16x32 tile of C and all of K, cut into blocks of 32 k; its 16 waves take
// the blocks in turn (wave w: blocks w, w + 16, w + 32, ...), so at any time
// the waves of every workgroup read one band of a few hundred consecutive
// rows of B and the whole chip streams B band by band. (With each wave
// owning one contiguous 1/16 of K instead, every workgroup reads 16 bands
// far apart, 128 bytes per row of each: on MI355X a cold 16 x 8192 x 8192
// call then read B at 3.9 TB/s, in the banded order at 5.0 TB/s.) B stored
// transposed keeps the contiguous runs: there a workgroup's 32 columns are
// one contiguous region of memory already. Each wave keeps two blocks in
// flight: the loads of its next block are issued before the MFMAs of the
// current one.
// Operands go straight from global memory into MFMA registers (no LDS tile):
// lane l of a wave reads rows k = 4*(l/16) + s of a 16-k step at column l%16
// of each 16-column block -- or, when B is read along N 8 bytes at a time,
// at columns 2(l%16) and 2(l%16) + 1, the two accumulators then holding the
// even and the odd columns -- and a 16-byte run of 4 consecutive k of row
// l%16 of A. At the end the 16 partial tiles are summed in a fixed order
// through LDS (deterministic) and the epilogue writes C.
// ===========================================================================
constexpr int SK_BM = 16, SK_BN = 32, SK_WAVES = 16, SK_KB = 32;  // k per block
#ifndef SGEMM_SKINNY_XCD
#define SGEMM_SKINNY_XCD 1
#endif

typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2 buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

template <bool VEC, bool TA = false, bool TB = false, bool TC = false>
__global__ __launch_bounds__(1024) void k_mfma_skinny(Args a, int tiles_m, int tiles_n, int xcd_remap) {
    // Rows padded to 68 floats: in the reduction below, the two 16-lane
    // halves of a half-wave read the two column blocks, 4 rows apart, which
    // the pad puts 16 banks apart (with 64 floats they shared banks).
    __shared__ float red[SK_WAVES][2][4][68];
    // With xcd_remap, neighbouring tiles on one XCD (workgroup i runs on XCD
    // i mod 8): two neighbours share the cache lines their rows of B straddle
    // when a row of B is not whole 128-byte lines, and one XCD's L2 then
    // fetches such a line once (see launch_skinny).
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, 1, xcd_remap != 0, tm, tn);
    const int m0 = __builtin_amdgcn_readfirstlane(tm * SK_BM), n0 = __builtin_amdgcn_readfirstlane(tn * SK_BN);
    const int rows_valid = (a.M - m0) < SK_BM ? (a.M - m0) : SK_BM;
    const int cols_valid = (a.N - n0) < SK_BN ? (a.N - n0) : SK_BN;
    // The wave index in a scalar register: the blocks a wave takes, and so
    // each block's buffer resources, derive from it, and a resource held in
    // vector registers costs a per-lane loop around every load.
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;

    // With both operands transposed and 4-byte loads, the addresses and
    // values of two blocks of 32 k exceed the 128 registers of a 1024-lane
    // workgroup: such calls take blocks of 16 k.
    constexpr int KB = (!VEC && TA && TB) ? SK_KB / 2 : SK_KB;
    const int nblocks = (a.K + KB - 1) / KB;
    struct Regs {
        f32x4 af[KB / 16];
        float b0[KB / 4], b1[KB / 4];
    };
    // PAIR: B is read along N 8 bytes at a time (see `pair` below): b0 holds
    // column 2c, b1 column 2c + 1; otherwise columns c and c + 16.
    auto load = [&](int blk, Regs& r, auto pair) {
        constexpr bool PAIR = decltype(pair)::value;
        // A block at or past the end of K (kk = 0) has empty resources:
        // every load reads zero and nothing is fetched.
        // (Wave-uniform; the clamps below compile to vector instructions,
        // and readfirstlane keeps the resources in scalar registers.)
        const int k0 = __builtin_amdgcn_readfirstlane(blk * KB);
        const int kr = a.K - k0;
        const int kk = __builtin_amdgcn_readfirstlane(kr <= 0 ? 0 : (kr < KB ? kr : KB));  // rows present
        const __amdgpu_buffer_rsrc_t rA =
            TA ? make_rsrc(a.A + (int64_t)k0 * a.lda + m0,
                           kk > 0 ? (uint32_t)(((int64_t)(kk - 1) * a.lda + rows_valid) * 4) : 0u)
               : make_rsrc(a.A + (int64_t)m0 * a.lda + k0,
                           kk > 0 ? (uint32_t)(((int64_t)(rows_valid - 1) * a.lda + kk) * 4) : 0u);
        const __amdgpu_buffer_rsrc_t rB =
            TB ? make_rsrc(a.B + (int64_t)n0 * a.ldb + k0,
                           kk > 0 ? (uint32_t)(((int64_t)(cols_valid - 1) * a.ldb + kk) * 4) : 0u)
               : make_rsrc(a.B + (int64_t)k0 * a.ldb + n0,
                           kk > 0 ? (uint32_t)(((int64_t)(kk - 1) * a.ldb + cols_valid) * 4) : 0u);
#pragma unroll
        for (int u = 0; u < KB / 16; ++u) {
            const int kq = 16 * u + 4 * g;  // this lane's 4 consecutive k
            if (VEC && !TA) {
                const bool ok = c < rows_valid && kq + 4 <= kk;
                r.af[u] = buf_load4(rA, ok ? (uint32_t)((c * (int)a.lda + kq) * 4) : OOB);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = c < rows_valid && kq + e < kk;
                    const int off = TA ? (kq + e) * (int)a.lda + c : c * (int)a.lda + kq + e;
                    r.af[u][e] = buf_load1(rA, ok ? (uint32_t)(off * 4) : OOB);
                }
            }
            if (VEC && TB) {
                // Columns c and c + 16 of B are rows of the stored matrix:
                // 4 consecutive k in one 16-byte load each.
                const bool ok = kq + 4 <= kk;
                const f32x4 x0 = buf_load4(rB, ok && c < cols_valid ? (uint32_t)((c * (int)a.ldb + kq) * 4) : OOB);
                const f32x4 x1 = buf_load4(rB, ok && c + 16 < cols_valid
                                                   ? (uint32_t)(((c + 16) * (int)a.ldb + kq) * 4) : OOB);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    r.b0[4 * u + e] = x0[e];
                    r.b1[4 * u + e] = x1[e];
                }
            } else if (PAIR) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kq_e = kq + e;
                    const f32x2 x = buf_load2(rB, kq_e < kk ? (uint32_t)((kq_e * (int)a.ldb + 2 * c) * 4) : OOB);
                    r.b0[4 * u + e] = x.x;
                    r.b1[4 * u + e] = x.y;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kq_e = kq + e;
                    const bool okr = kq_e < kk;
                    const int o0 = TB ? c * (int)a.ldb + kq_e : kq_e * (int)a.ldb + c;
                    const int o1 = TB ? (c + 16) * (int)a.ldb + kq_e : kq_e * (int)a.ldb + c + 16;
                    r.b0[4 * u + e] = buf_load1(rB, okr && c < cols_valid ? (uint32_t)(o0 * 4) : OOB);
                    r.b1[4 * u + e] = buf_load1(rB, okr && c + 16 < cols_valid ? (uint32_t)(o1 * 4) : OOB);
                }
            }
        }
    };
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
    auto mma = [&](const Regs& r) {
#pragma unroll
        for (int u = 0; u < KB / 16; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(r.af[u][e], r.b0[4 * u + e], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(r.af[u][e], r.b1[4 * u + e], acc1, 0, 0, 0);
            }
    };
    // This wave's blocks (w, w + 16, ...: see BANDED), two in flight: the
    // loads of its next block go out before the MFMAs of the current one
    // (register sets r0, r1). The
    // loads are unconditional (past the end of K they read zeros), and
    // scheduling fences keep each block's loads ahead of the other block's
    // MFMAs: loads issued on only some paths, or sunk below the MFMAs, make
    // the compiler wait for every load in flight, the prefetched ones
    // included, before a block's MFMAs.
    // With B stored transposed a workgroup's 32 columns are 32 whole rows
    // of the stored matrix, one contiguous region, which streams best with
    // each wave taking one contiguous run of blocks instead (wave w: blocks
    // w * per .. w * per + per - 1).
    constexpr bool BANDED = !TB;
    const int per = (nblocks + SK_WAVES - 1) / SK_WAVES;
    const int count = BANDED ? (nblocks > w ? (nblocks - w + SK_WAVES - 1) / SK_WAVES : 0)
                             : (nblocks - w * per < per ? (nblocks - w * per > 0 ? nblocks - w * per : 0) : per);
    // The wave's i-th block; past its last one, a block past the end of K.
    auto blk = [&](int i) { return i >= count ? nblocks : BANDED ? w + SK_WAVES * i : w * per + i; };
    auto run = [&](auto pair) {
        Regs r0, r1;
        load(blk(0), r0, pair);
        for (int i = 0; i < count; i += 2) {
            load(blk(i + 1), r1, pair);
            __builtin_amdgcn_sched_barrier(0);
            mma(r0);
            __builtin_amdgcn_sched_barrier(0);
            load(blk(i + 2), r0, pair);
            __builtin_amdgcn_sched_barrier(0);
            if (i + 1 < count) mma(r1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Pair reads need untransposed B with 8-byte aligned rows and a tile
    // wholly inside N (at the edge a pair would straddle the last column).
    const bool pair = !TB && VEC && (a.ldb & 1) == 0 && ((uintptr_t)a.B & 7) == 0 && cols_valid == SK_BN;
    if (pair)
        run(std::true_type{});
    else
        run(std::false_type{});

#pragma unroll
    for (int r = 0; r < 4; ++r) {
        red[w][0][r][lane] = acc0[r];
        red[w][1][r][lane] = acc1[r];
    }
    __syncthreads();
    if (threadIdx.x < SK_BM * SK_BN) {
        // Consecutive threads take consecutive columns of a row-major C, or
        // consecutive rows of a column-major one (TC).
        const int i = TC ? threadIdx.x % SK_BM : threadIdx.x / SK_BN;
        const int j = TC ? threadIdx.x / SK_BM : threadIdx.x % SK_BN;
        const int bj = pair ? (j & 1) : (j >> 4), cj = pair ? (j >> 1) : (j & 15);
        const int src = (i >> 2) * 16 + cj, r = i & 3;
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < SK_WAVES; ++ww) v += red[ww][bj][r][src];
        if (i < rows_valid && j < cols_valid) {
            if (TC)
                store_out_col(a, (int64_t)m0 + i, (int64_t)n0 + j, v);
            else
                store_out(a, (int64_t)m0 + i, (int64_t)n0 + j, v);
        }
    }
}

static int check_skinny(const Args& a) {
    const int64_t ea = extent_a(a, SK_BM, SK_KB);
    const int64_t eb = extent_b(a, SK_KB, SK_BN);
    if (ea >= (int64_t)OOB || eb >= (int64_t)OOB) return SGEMM_F32_ERR_TOO_LARGE;
    const int64_t tiles = cdiv(a.M, SK_BM) * cdiv(a.N, SK_BN);
    return tiles <= max_workgroups(1024) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
}

static hipError_t launch_skinny(const Args& a, hipStream_t s) {
    const int tm = (int)cdiv(a.M, SK_BM), tn = (int)cdiv(a.N, SK_BN);
    const dim3 grid((unsigned)(tm * tn)), block(1024);
    // Neighbouring tiles on one XCD when B's rows straddle 128-byte lines
    // (a pitch or base that is not whole lines) or B is read transposed:
    // 16x8191x8192 73.1 -> 43.4 us back to back, 8192x16x8192 (the few-column
    // product, run transposed) 51.5 -> 45.8, B transposed 52.8 -> 50.1. With
    // whole lines of an untransposed B the workgroups stay in dispatch order,
    // which streams a cold B 3% faster (16x8192x8192 53.2 against 54.8 us).
    const bool partial_lines = a.tb || (a.ldb & 31) || ((uintptr_t)a.B & 127);
    const int xr = (SGEMM_SKINNY_XCD && partial_lines) ? xcd_remap_enabled() : 0;
    const bool vec = small_vec_ok(a);
    return with_trans(a, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        if (a.tc) {
            if (vec)
                hipLaunchKernelGGL((k_mfma_skinny<true, TA, TB, true>), grid, block, 0, s, a, tm, tn, xr);
            else
                hipLaunchKernelGGL((k_mfma_skinny<false, TA, TB, true>), grid, block, 0, s, a, tm, tn, xr);
        } else if (vec) {
            hipLaunchKernelGGL((k_mfma_skinny<true, TA, TB>), grid, block, 0, s, a, tm, tn, xr);
        } else {
            hipLaunchKernelGGL((k_mfma_skinny<false, TA, TB>), grid, block, 0, s, a, tm, tn, xr);
        }
        return hipGetLastError();
    });
}

Variant kMfmaSkinny = {"mfma_skinny", check_skinny, launch_skinny,
                       (const void*)k_mfma_skinny<true>, 1024, true};

}  // namespace sgemm
