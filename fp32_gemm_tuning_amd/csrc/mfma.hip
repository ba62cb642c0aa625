// FP32 matrix-core SGEMM kernels for gfx950 (true FP32 MFMA: FP32 operands,
// FP32 accumulate; no reduced-precision input types).
//
// SGEMM is a dense contraction, so on CDNA4 it belongs on the matrix cores:
// v_mfma_f32_32x32x2_f32 multiplies a 32x2 by a 2x32 block and accumulates a
// 32x32 block (4096 FLOP per wave instruction); v_mfma_f32_16x16x4_f32 does
// 16x4 by 4x16 into 16x16 (2048 FLOP). The pages' CUDA-core ladder (block
// tile in shared memory, per-thread register patch, double buffering; see
// "Optimizing Matrix Multiply on CUDA, Part 2", "Overlapping Loads and
// Computation") maps onto this as: block tile in LDS, per-wave accumulator
// blocks held in registers, one MFMA per (row block, column block, k pair).
//
// Operand layouts (one wave, lane l):
//   32x32x2: A operand lane l = A[l%32][l/32], B operand = B[l/32][l%32],
//            result register r of lane l = C[8*(r/4) + 4*(l/32) + r%4][l%32].
//   16x16x4: A operand lane l = A[l%16][l/16], B operand = B[l/16][l%16],
//            result register r of lane l = C[4*(l/16) + r][l%16].
// The k index inside one MFMA is only a summation index, so each half (or
// quarter) of the wave walks its own contiguous run of k: in a BK-deep slice
// lane l feeds the instruction's k slot l/32 (l/16) from k = BK/2*(l/32) + s
// (BK/4*(l/16) + s) at step s. A lane's A values for a slice are then BK/2
// (BK/4) consecutive floats of one row of the untransposed A tile, read with
// 16-byte LDS loads, and no transposed copy of A is needed; the B values are
// single floats of one row of the B tile, consecutive across lanes.
//
// Edges: every global read goes through a buffer resource; masked elements
// get an out-of-range offset and read as zero, so partial tiles need no
// branches in the K loop; only the final stores are guarded.
#include "kernels.hpp"

#include <type_traits>
#include "sgemm_f32.h"

namespace sgemm {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The LDS tile fill of one K slice: global -> registers (issued early), then
// registers -> LDS after the current slice's math. VEC: 16-byte chunks (needs
// K, N, lda, ldb multiples of 4 and 16-byte aligned A, B); otherwise 4-byte
// elements with per-element masks.
template <int BM, int BN, int BK, int NT, bool VEC>
struct TileFill {
    static constexpr int BNP = BN + 4;  // B tile pitch in floats
    static constexpr int CPR = BK / 4;  // 16-byte chunks per A row
    static constexpr int A_ELEMS = BM * BK / NT;   // floats of A per lane per slice
    static constexpr int B_ELEMS = BK * BN / NT;
    static_assert(A_ELEMS % 4 == 0 && B_ELEMS % 4 == 0, "tile/threads mismatch");

    f32x4 ra[A_ELEMS / 4];
    f32x4 rb[B_ELEMS / 4];

    // Global -> registers for slice starting at k0.
    __device__ __forceinline__ void load(const Args& a, int t, int m0, int n0, int k0,
                                         int rows_valid, int cols_valid) {
        const int kk = (a.K - k0) < BK ? (a.K - k0) : BK;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(
            a.A + (int64_t)m0 * a.lda + k0, (uint32_t)(((int64_t)(rows_valid - 1) * a.lda + kk) * 4));
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(
            a.B + (int64_t)k0 * a.ldb + n0, (uint32_t)(((int64_t)(kk - 1) * a.ldb + cols_valid) * 4));
        if (VEC) {
#pragma unroll
            for (int p = 0; p < A_ELEMS / 4; ++p) {
                const int c = t + NT * p, row = c / CPR, q = c % CPR;
                const bool ok = row < rows_valid && 4 * q + 4 <= kk;
                ra[p] = buf_load4(rA, ok ? (uint32_t)((row * (int)a.lda + 4 * q) * 4) : OOB);
            }
#pragma unroll
            for (int p = 0; p < B_ELEMS / 4; ++p) {
                const int c = t + NT * p, krow = c / (BN / 4), nq = c % (BN / 4);
                const bool ok = krow < kk && 4 * nq + 4 <= cols_valid;
                rb[p] = buf_load4(rB, ok ? (uint32_t)((krow * (int)a.ldb + 4 * nq) * 4) : OOB);
            }
        } else {
#pragma unroll
            for (int p = 0; p < A_ELEMS; ++p) {
                const int e = t + NT * p, row = e / BK, kq = e % BK;
                const bool ok = row < rows_valid && kq < kk;
                ra[p >> 2][p & 3] = buf_load1(rA, ok ? (uint32_t)((row * (int)a.lda + kq) * 4) : OOB);
            }
#pragma unroll
            for (int p = 0; p < B_ELEMS; ++p) {
                const int e = t + NT * p, krow = e / BN, n = e % BN;
                const bool ok = krow < kk && n < cols_valid;
                rb[p >> 2][p & 3] = buf_load1(rB, ok ? (uint32_t)((krow * (int)a.ldb + n) * 4) : OOB);
            }
        }
    }

    // Registers -> LDS. As: BM rows of BK floats, 16-byte chunk q of row r at
    // chunk q ^ swz_chunk<BK>(r). Bs: BK rows of BN floats at pitch BNP.
    __device__ __forceinline__ void store(float* As, float* Bs, int t) const {
        if (VEC) {
#pragma unroll
            for (int p = 0; p < A_ELEMS / 4; ++p) {
                const int c = t + NT * p, row = c / CPR, q = c % CPR;
                *(f32x4*)&As[row * BK + ((q ^ swz_chunk<BK>(row)) << 2)] = ra[p];
            }
#pragma unroll
            for (int p = 0; p < B_ELEMS / 4; ++p) {
                const int c = t + NT * p, krow = c / (BN / 4), nq = c % (BN / 4);
                *(f32x4*)&Bs[krow * BNP + 4 * nq] = rb[p];
            }
        } else {
#pragma unroll
            for (int p = 0; p < A_ELEMS; ++p) {
                const int e = t + NT * p, row = e / BK, kq = e % BK;
                As[row * BK + ((((kq >> 2) ^ swz_chunk<BK>(row)) << 2) | (kq & 3))] = ra[p >> 2][p & 3];
            }
#pragma unroll
            for (int p = 0; p < B_ELEMS; ++p) {
                const int e = t + NT * p, krow = e / BN, n = e % BN;
                Bs[krow * BNP + n] = rb[p >> 2][p & 3];
            }
        }
    }
};

// The same fill with gfx950's buffer-to-LDS loads: no prefetch registers and
// no LDS store instructions; a wave instruction writes 64 x 16 bytes (VEC) or
// 64 x 4 bytes contiguously, so each lane computes which global element
// belongs at its destination slot.
//
// One operand's part of a K slice is ROWS rows (along M for A, along N for
// B) by BK values of k. Its LDS layout follows its memory layout, so that
// every load moves whole 16-byte (or 4-byte) pieces:
//  - k-contiguous operands (A as stored, or a transposed B) keep [row][k]: BK
//    floats per row, 16-byte chunk q of row r at chunk q ^ swz_chunk<BK>(r)
//    (the lane inverts the swizzle); fragments are read 16 bytes at a time;
//  - row-contiguous operands (B as stored, or a transposed A) keep [k][row]:
//    ROWS floats per k, unpadded; fragments are read 4 bytes at a time, which
//    the LDS serves one half-wave at a time, each half reading 32
//    consecutive floats of one row.
// Element (row, k) of the slice starting at k0 is X[(r0 + row)*ld + k0 + k]
// in memory when the operand is k-contiguous, else X[(k0 + k)*ld + r0 + row].
// Wave w issues pieces w, w + W, w + 2W, ... of the TOTAL per slice, so the
// per-wave counts differ by at most one when W does not divide TOTAL.
template <int ROWS, int BK, int NT, bool VEC, bool KCONTIG>
struct OperandFill {
    static constexpr int W = NT / 64;
    static constexpr int EPI = VEC ? 256 : 64;   // floats per wave instruction
    static constexpr int TOTAL = ROWS * BK / EPI;
    static_assert(TOTAL * EPI == ROWS * BK, "tile/instruction mismatch");
    static constexpr int INSTR = (TOTAL + W - 1) / W;   // per wave per slice, at most
    static constexpr bool EVEN = TOTAL % W == 0;
    static constexpr int CPR = BK / 4;                  // 16-byte chunks per k-contiguous row

    // A slice starting at or past K is legal: its resource is empty and every
    // lane's load reads as zero (the pipelined kernel issues loads for slices
    // past the end so that every path issues the same number). FULL: the
    // tile lies wholly inside the matrix and K is a multiple of BK, so no lane
    // needs a range mask (16-byte loads only).
    template <bool FULL>
    __device__ __forceinline__ void issue(const float* X, int64_t ld, int r0, int k0, int K,
                                          int rows_valid, int t, float* dst_base) const {
        // kk = valid k in the slice (0 past the end): then no lane is in
        // range, and the extents stay below 2^31 bytes, so the out-of-range
        // offset always reads zero. The base address may point past the
        // matrix; nothing is read through it. With FULL a slice is whole or
        // past the end, a choice the scalar unit makes; the general clamp
        // compiles to a vector instruction, and readfirstlane keeps the
        // resource in scalar registers.
        const int kr = K - k0;
        const int kk = FULL ? (kr > 0 ? BK : 0)
                            : __builtin_amdgcn_readfirstlane(kr <= 0 ? 0 : (kr < BK ? kr : BK));
        __amdgpu_buffer_rsrc_t r;
        if (KCONTIG)
            r = make_rsrc(X + (int64_t)r0 * ld + k0,
                          (FULL && kk == 0) ? 0u : (uint32_t)(((int64_t)(rows_valid - 1) * ld + kk) * 4));
        else
            r = make_rsrc(X + (int64_t)k0 * ld + r0,
                          kk > 0 ? (uint32_t)(((int64_t)(kk - 1) * ld + rows_valid) * 4) : 0u);
        const int ldi = (int)ld;
        const int w = t >> 6, lane = t & 63;
#pragma unroll
        for (int p = 0; p < INSTR; ++p) {
            const int piece = w + W * p;
            if (!EVEN && piece >= TOTAL) break;
            const float* dst = dst_base + piece * EPI;
            if (KCONTIG && VEC) {
                const int slot = piece * 64 + lane;       // 16-byte chunk index in the tile
                const int row = slot / CPR, q = (slot % CPR) ^ swz_chunk<BK>(row);
                const bool ok = FULL || (row < rows_valid && 4 * q + 4 <= kk);
                buf_load_lds16(r, dst, ok ? (uint32_t)((row * ldi + 4 * q) * 4) : OOB);
            } else if (KCONTIG) {
                const int f = piece * 64 + lane;          // float index in the tile
                const int row = f / BK, pc = (f % BK) >> 2;
                const int kq = ((pc ^ swz_chunk<BK>(row)) << 2) | (f & 3);
                const bool ok = row < rows_valid && kq < kk;
                buf_load_lds4(r, dst, ok ? (uint32_t)((row * ldi + kq) * 4) : OOB);
            } else if (VEC) {
                const int slot = piece * 64 + lane;
                const int krow = slot / (ROWS / 4), nq = slot % (ROWS / 4);
                const bool ok = FULL || (krow < kk && 4 * nq + 4 <= rows_valid);
                buf_load_lds16(r, dst, ok ? (uint32_t)((krow * ldi + 4 * nq) * 4) : OOB);
            } else {
                const int f = piece * 64 + lane;
                const int krow = f / ROWS, n = f % ROWS;
                const bool ok = krow < kk && n < rows_valid;
                buf_load_lds4(r, dst, ok ? (uint32_t)((krow * ldi + n) * 4) : OOB);
            }
        }
    }
};

// Both operands of a slice. TA / TB: the operand is stored transposed (A as
// K x M, B as N x K, row-major), which makes A row-contiguous and B
// k-contiguous.
template <int BM, int BN, int BK, int NT, bool VEC, bool TA = false, bool TB = false>
struct TileFillDma {
    using FA = OperandFill<BM, BK, NT, VEC, !TA>;
    using FB = OperandFill<BN, BK, NT, VEC, TB>;
    static constexpr int BNP = BN;
    static constexpr int A_INSTR = FA::INSTR, B_INSTR = FB::INSTR;
    static constexpr bool EVEN = FA::EVEN && FB::EVEN;

    template <bool FULL = false>
    __device__ __forceinline__ void issue(const Args& a, int t, int m0, int n0, int k0,
                                          int rows_valid, int cols_valid, float* As,
                                          float* Bs) const {
        FA().template issue<FULL>(a.A, a.lda, m0, k0, a.K, rows_valid, t, As);
        FB().template issue<FULL>(a.B, a.ldb, n0, k0, a.K, cols_valid, t, Bs);
    }
};

// One wave's share of a BK-deep slice held in LDS, multiplied in 16-deep
// sub-steps with v_mfma_f32_32x32x2_f32: in sub-step u, lanes 0-31 (h = 0)
// take k = 16u + s and lanes 32-63 take k = 16u + 8 + s at MFMA step
// s = 0..7, so each lane needs 8 consecutive k of its row (of A) and of its
// column (of B). A k-contiguous stage ([row][k] with the XOR chunk swizzle:
// A, or B stored transposed) yields them in two 16-byte reads at chunks
// 4u + 2h and 4u + 2h + 1; a row-contiguous one ([k][row]: B, or A stored
// transposed) in 8 4-byte reads down rows 16u + 8h .. 16u + 8h + 7. The
// offsets are in floats from the stage base plus abase / bbase.
template <int BM, int BN, int WM, int WN, int BK, bool TA, bool TB>
struct SubstepMma {
    static constexpr int STEPS = BK / 16, BI = WM / 32, BJ = WN / 32;
    int aoff[STEPS][BI][2], boff[STEPS][BJ][2];

    __device__ __forceinline__ SubstepMma(int wm, int wn, int h, int c, int abase, int bbase) {
#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
#pragma unroll
            for (int bi = 0; bi < BI; ++bi) {
                const int row = wm * WM + bi * 32 + c;
#pragma unroll
                for (int v = 0; v < 2; ++v)
                    aoff[u][bi][v] = TA ? abase + (16 * u + 8 * h) * BM + row
                                        : abase + row * BK + (((4 * u + 2 * h + v) ^ swz_chunk<BK>(row)) << 2);
            }
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj) {
                const int col = wn * WN + bj * 32 + c;
#pragma unroll
                for (int v = 0; v < 2; ++v)
                    boff[u][bj][v] = TB ? bbase + col * BK + (((4 * u + 2 * h + v) ^ swz_chunk<BK>(col)) << 2)
                                        : bbase + (16 * u + 8 * h) * BN + col;
            }
        }
    }

    template <bool KCONTIG, int PITCH>
    static __device__ __forceinline__ void frag8(const float* X, const int (&off)[2], float (&f)[8]) {
        if (KCONTIG) {
            const f32x4 lo = *(const f32x4*)&X[off[0]];
            const f32x4 hi = *(const f32x4*)&X[off[1]];
            f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
            f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) f[k] = X[off[0] + k * PITCH];
        }
    }

    __device__ __forceinline__ void operator()(const float* Ac, const float* Bc,
                                               f32x16 (&acc)[BI][BJ]) const {
#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
            float af[BI][8], bf[BJ][8];
#pragma unroll
            for (int bi = 0; bi < BI; ++bi) frag8<!TA, BM>(Ac, aoff[u][bi], af[bi]);
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj) frag8<TB, BN>(Bc, boff[u][bj], bf[bj]);
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                    for (int bj = 0; bj < BJ; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[bi][k], bf[bj][k],
                                                                           acc[bi][bj], 0, 0, 0);
        }
    }
};

// ===========================================================================
// Tile parameters of mfma_128x128 and mfma_64x128, two instances of the
// pipelined kernel below (k_mfma_pipe), set at compile time so that the
// autotuner (fp32_gemm_tuning_amd/autotune.py) can sweep them. mfma_128x128
// is BM = BN = 128 with 8 waves of 64x32 (32 accumulator registers per
// lane), BK = 32, and an occupancy target of 4 waves per SIMD (2 workgroups
// per compute unit); mfma_64x128 is 64x128 with 4 waves of 64x32, BK = 32
// and 3 workgroups per compute unit. The block and wave tiles came from a sweep of the earlier
// single-buffered tile kernel on MI355X; moved onto the pipelined kernel
// they gain 3-20% (2048^3 122.6 -> 130.5, 512x4096x4096 108.8 -> 130.5
// TFLOP/s) and lose 4% only on the 1000x1531x777 odd shape, which the
// dispatch gives to a K-group kernel.
// ===========================================================================
#ifndef SGEMM_M128_BK
#define SGEMM_M128_BK 32
#endif
#ifndef SGEMM_M128_WAVES_PER_EU
#define SGEMM_M128_WAVES_PER_EU 4
#endif
#ifndef SGEMM_M128_BM
#define SGEMM_M128_BM 128
#endif
#ifndef SGEMM_M128_BN
#define SGEMM_M128_BN 128
#endif
#ifndef SGEMM_M128_WM
#define SGEMM_M128_WM 64
#endif
#ifndef SGEMM_M128_WN
#define SGEMM_M128_WN 32
#endif
#ifndef SGEMM_M128_GROUP_M
#define SGEMM_M128_GROUP_M 8
#endif
#ifndef SGEMM_M64x128_WM
#define SGEMM_M64x128_WM 64
#endif
#ifndef SGEMM_M64x128_WN
#define SGEMM_M64x128_WN 32
#endif
#ifndef SGEMM_M64x128_BK
#define SGEMM_M64x128_BK 32
#endif
constexpr int M128_BM = SGEMM_M128_BM, M128_BN = SGEMM_M128_BN, M128_BK = SGEMM_M128_BK;
constexpr int M128_WM = SGEMM_M128_WM, M128_WN = SGEMM_M128_WN, M128_GROUP_M = SGEMM_M128_GROUP_M;

// ---------------------------------------------------------------------------
// Stream-K (SkPlan in common.hpp). A run of slices that covers a whole tile
// writes C directly; any other run leaves its partial tile in the workspace,
// and a second kernel on the same stream (k_sk_fixup) sums the pieces of
// each split tile in K order -- so the result does not depend on which
// piece finished first -- and writes C. The kernel boundary orders the
// partial stores before their reads. (The pages let the unit that computes
// a tile's last piece combine the pieces inside the one kernel. On MI355X
// that needs a release fence per piece and an acquire per tile at device
// scope, and each of those writes back or invalidates a whole XCD's L2,
// which cost 13-37 us per call at 1536^3-3072^3, against a few us for the
// second launch.)
//
// Partial tiles travel as 16-byte vectors: vector q of thread t of a BM x BN
// tile is at float offset (q * NT + t) * 4 of its slot, so each access of a
// wave is 1 KiB contiguous, and the fixup kernel, with the same thread
// layout, reads back exactly the values each of its threads owns.
// ---------------------------------------------------------------------------
template <int BI, int BJ, int NT>
struct PartialIo {
    static constexpr int Q = BI * BJ * 4;   // 16-byte vectors per lane

    __device__ __forceinline__ static void put(float* slot, int t, const f32x16 (&acc)[BI][BJ]) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int bi = q / (4 * BJ), bj = (q / 4) % BJ, r0 = (q % 4) * 4;
            *(f32x4*)(slot + ((size_t)q * NT + t) * 4) =
                f32x4{acc[bi][bj][r0], acc[bi][bj][r0 + 1], acc[bi][bj][r0 + 2], acc[bi][bj][r0 + 3]};
        }
    }

    // acc = slot (FIRST) or acc += slot, one 32x32 block at a time (the asm
    // pin keeps the compiler from loading a whole partial tile at once).
    template <bool FIRST>
    __device__ __forceinline__ static void gather(const float* slot, int t, f32x16 (&acc)[BI][BJ]) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int bi = q / (4 * BJ), bj = (q / 4) % BJ, r0 = (q % 4) * 4;
            const f32x4 v = *(const f32x4*)(slot + ((size_t)q * NT + t) * 4);
            if (FIRST) {
                acc[bi][bj][r0] = v.x;
                acc[bi][bj][r0 + 1] = v.y;
                acc[bi][bj][r0 + 2] = v.z;
                acc[bi][bj][r0 + 3] = v.w;
            } else {
                acc[bi][bj][r0] += v.x;
                acc[bi][bj][r0 + 1] += v.y;
                acc[bi][bj][r0 + 2] += v.z;
                acc[bi][bj][r0 + 3] += v.w;
            }
            if (q % 4 == 3) asm volatile("" : "+v"(acc[bi][bj])::"memory");
        }
    }
};

// Slot of workgroup jj's piece of split tile st: its first run (slot 2jj)
// if that run starts in the tile, else its last run (slot 2jj+1).
__device__ __forceinline__ int sk_slot(const SkPlan& p, int jj, int st) {
    return (jj * p.upw >= st * p.slices) ? 2 * jj : 2 * jj + 1;
}

// ===========================================================================
// The same tile with a software-pipelined slice and an LDS ring of STAGES
// slices. Each BK = 16 slice is split into two halves of four MFMA k-steps,
// and every wave holds two fragment register sets, so the LDS reads of one
// half are in flight while the MFMAs of the other half run. The workgroup
// barrier sits between the two halves of a slice: before it, each wave has
// finished reading the slice's stage and its own buffer-to-LDS loads of the
// next slice have landed (loads of later slices may still be in flight);
// after it, the loads of the slice STAGES ahead are issued into the stage
// just released, and the first half of the next slice is read while the
// second half of this one is multiplied. A lone wave on a SIMD then never
// waits on an LDS round trip between MFMAs, and a global load has STAGES - 1
// slices of time to land.
// ===========================================================================
// The instruction order within one scheduling region of the pipelined slice:
// a part's MFMAs with the LDS fragment reads of the next part woven in, one
// read after every two MFMAs, and, with LOADS > 0, that many of the slice's
// buffer-to-LDS loads spread over the region, each after a group of three
// reads. Issued in one burst right after the workgroup barrier, the reads of
// sixteen waves fill the LDS command queue, and the loads' scalar set-up
// holds every wave of a SIMD at once; woven in, a ready MFMA is always at
// hand (about 2.5% at 4096^3 and 8192^3, bit-identical results: the MFMA
// order per accumulator is unchanged). Instructions past the pattern's counts
// (the transposed and 4-byte-fill instances read and load more) are placed
// by the scheduler.
template <int LOADS>
__device__ __forceinline__ void weave_half() {
    constexpr int MFMA = 0x008, VMEM_READ = 0x020, DS_READ = 0x100;
    if constexpr (LOADS == 0) {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            __builtin_amdgcn_sched_group_barrier(MFMA, 2, 0);
            __builtin_amdgcn_sched_group_barrier(DS_READ, 1, 0);
        }
    } else {
#pragma unroll
        for (int l = 0; l < LOADS; ++l) {
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                __builtin_amdgcn_sched_group_barrier(MFMA, 2, 0);
                __builtin_amdgcn_sched_group_barrier(DS_READ, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(VMEM_READ, 1, 0);
        }
    }
    __builtin_amdgcn_sched_group_barrier(MFMA, 64, 0);   // the rest
}

template <int BI, int BJ>
struct PartFrag {
    f32x4 a[BI];      // A operands of the part's 4 k-steps, per row block
    float b[BJ][4];   // B operands of the part's 4 k-steps, per column block
};

// Workgroup barrier of the LDS ring: waits until at most VMCNT of this wave's
// vector-memory operations (buffer-to-LDS loads of later slices, issued after
// the ones that must have landed) are outstanding and all of its LDS reads
// are done, then synchronises the workgroup. A fence would wait for every
// outstanding load, so the compiler is instead kept from moving memory
// accesses across the barrier by empty asm statements with a memory clobber.
// s_waitcnt immediate (gfx9): vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8.
template <int VMCNT>
__device__ __forceinline__ void ring_barrier() {
    static_assert(VMCNT >= 0 && VMCNT < 64, "vmcnt field is 6 bits");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((VMCNT & 15) | ((VMCNT >> 4) << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The body of k_mfma_pipe, shared with its stream-K form: the product of
// slices [s_begin, s_end) of one tile through the LDS ring, and the
// epilogue. On return every load issued into the ring has landed and every
// wave has passed the last barrier, so the ring may be refilled.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, bool VEC, bool FULL, bool TA,
          bool TB>
struct PipeCore {
    static_assert(BK == 16 || BK == 32, "slices of 16 or 32 k");
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0,
                  "wave tiles are whole 32x32 blocks that divide the block tile");
    static_assert((BM / WM) * (BN / WN) * 64 <= 1024, "at most 16 waves per workgroup");
    static constexpr int P = BK / 8;   // parts of 4 MFMA k-steps per slice
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NT = (BM / WM) * WAVES_N * 64;
    static constexpr int BI = WM / 32, BJ = WN / 32;
    using Dma = TileFillDma<BM, BN, BK, NT, VEC, TA, TB>;
    static constexpr int BNP = Dma::BNP, APITCH = BK;
    // Deeper rings count outstanding loads, which must then be the same on
    // every wave; with two stages the barrier waits for all of them.
    static_assert(Dma::EVEN || STAGES == 2, "the ring barrier counts the same loads on every wave");
    static constexpr int G = Dma::A_INSTR + Dma::B_INSTR;   // loads per wave per slice
    static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 LDS stages");
    static_assert((STAGES - 2) * G < 64, "outstanding loads exceed vmcnt");
    // The prologue leaves the later stages' loads in flight only when every
    // wave issues the same G loads per slice (G is the largest per-wave
    // count; a wave that issues fewer must wait for all of its own) and the
    // count fits the 6-bit field.
    static constexpr int PROLOGUE_VMCNT = (Dma::EVEN && (STAGES - 1) * G < 64) ? (STAGES - 1) * G : 0;
    static constexpr int LDS_A = BM * APITCH, LDS_B = BK * BNP;

    int m0, n0, rows_valid, cols_valid, t, wm, wn, h, c;

    __device__ __forceinline__ PipeCore(const Args& a, int tm, int tn, int tid = threadIdx.x) {
        // The tile coordinates are workgroup-uniform; the integer divisions
        // of the tile mapping leave them in vector registers, and a buffer
        // resource built from a vector register costs a per-lane loop around
        // every load, so move them to scalar registers explicitly.
        m0 = __builtin_amdgcn_readfirstlane(tm * BM);
        n0 = __builtin_amdgcn_readfirstlane(tn * BN);
        rows_valid = (a.M - m0) < BM ? (a.M - m0) : BM;
        cols_valid = (a.N - n0) < BN ? (a.N - n0) : BN;
        t = tid;
        const int lane = t & 63, w = t >> 6;
        wm = w / WAVES_N;
        wn = w % WAVES_N;
        h = lane >> 5;
        c = lane & 31;
    }

    __device__ __forceinline__ static void zero(f32x16 (&acc)[BI][BJ]) {
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
            for (int j = 0; j < BJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    }

    __device__ __forceinline__ void mainloop(const Args& a, int s_begin, int s_end,
                                             float* const (&Ast)[4], float* const (&Bst)[4],
                                             f32x16 (&acc)[BI][BJ]) const {
        // Lanes 0-31 take k = s and lanes 32-63 take k = BK/2 + s at MFMA step s
        // of the slice; part v covers steps 4v .. 4v+3, i.e. 16-byte chunk
        // P*h + v of a k-contiguous row ([row][k], swizzled: A, or B stored
        // transposed) and rows BK/2*h + 4v .. BK/2*h + 4v + 3 of a row-contiguous
        // stage ([k][row]: B, or A stored transposed). A chunk address of part v
        // is xrow + ((xchunk ^ v) << 2), computed per read (one XOR and one
        // shift-or, hidden under the MFMAs) rather than held in P registers per
        // block.
        int arow[BI], achunk[BI], brow[BJ], bchunk[BJ];
#pragma unroll
        for (int bi = 0; bi < BI; ++bi) {
            const int row = wm * WM + bi * 32 + c;
            arow[bi] = TA ? (BK / 2) * h * BM + row : row * APITCH;
            achunk[bi] = (P * h) ^ swz_chunk<BK>(row);
        }
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj) {
            const int col = wn * WN + bj * 32 + c;
            brow[bj] = TB ? col * BK : (BK / 2) * h * BNP + col;
            bchunk[bj] = (P * h) ^ swz_chunk<BK>(col);
        }

        auto read_part = [&](PartFrag<BI, BJ>& f, const float* Ac, const float* Bc, int v) {
#pragma unroll
            for (int bi = 0; bi < BI; ++bi) {
                if constexpr (TA) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) f.a[bi][k] = Ac[arow[bi] + (4 * v + k) * BM];
                } else {
                    f.a[bi] = *(const f32x4*)&Ac[arow[bi] + ((achunk[bi] ^ v) << 2)];
                }
            }
            if constexpr (TB) {
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj) {
                    const f32x4 q = *(const f32x4*)&Bc[brow[bj] + ((bchunk[bj] ^ v) << 2)];
                    f.b[bj][0] = q.x; f.b[bj][1] = q.y; f.b[bj][2] = q.z; f.b[bj][3] = q.w;
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int bj = 0; bj < BJ; ++bj) f.b[bj][k] = Bc[brow[bj] + (4 * v + k) * BNP];
            }
        };
        auto mma_part = [&](const PartFrag<BI, BJ>& f, int k_begin = 0, int k_end = 4) {
#pragma unroll
            for (int k = k_begin; k < k_end; ++k)
#pragma unroll
                for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                    for (int bj = 0; bj < BJ; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[bi][k], f.b[bj][k],
                                                                           acc[bi][bj], 0, 0, 0);
        };

        const Dma dma;
        PartFrag<BI, BJ> f0, f1;
        // Prologue: fill every stage (stages past the last slice read zeros),
        // wait for slice 0, read its first half. Every slice below issues exactly
        // G loads per wave, whether or not its target slice exists, so the count
        // of loads issued after any given one is the same on every path.
#pragma unroll
        for (int j = 0; j < STAGES; ++j)
            dma.template issue<FULL>(a, t, m0, n0, (s_begin + j) * BK, rows_valid, cols_valid, Ast[j],
                                     Bst[j]);
        ring_barrier<PROLOGUE_VMCNT>();
        read_part(f0, Ast[0], Bst[0], 0);

        // Slice s lives in stage (Ac, Bc), slice s + 1 in (An, Bn); on entry f0
        // holds (or is loading) part 0 of slice s; parts alternate between f0
        // and f1 (P is even, so the last part is in f1). The barrier comes after
        // the reads of the last part and before its MFMAs; at the barrier the
        // loads of slices s + 2 .. s + STAGES - 1 may still be in flight.
        // Each part's MFMAs form one scheduling region with the reads of the
        // next part (and, after the barrier, the loads of slice s + STAGES),
        // ordered by weave_half; scheduling fences keep the regions apart (the
        // scheduler would otherwise hoist the barrier, with its wait on the
        // reads just issued, above the MFMAs, or pull MFMAs up next to the
        // reads they depend on).
        auto slice = [&](int s, float* Ac, float* Bc, const float* An, const float* Bn) {
#pragma unroll
            for (int v = 0; v + 1 < P; ++v) {
                if (v & 1)
                    read_part(f0, Ac, Bc, v + 1);
                else
                    read_part(f1, Ac, Bc, v + 1);
                if (v & 1)
                    mma_part(f1);
                else
                    mma_part(f0);
                weave_half<0>();
                __builtin_amdgcn_sched_barrier(0);
            }
            ring_barrier<(STAGES - 2) * G>();
            read_part(f0, An, Bn, 0);   // past the last slice: read and unused
            mma_part(f1);
            dma.template issue<FULL>(a, t, m0, n0, (s + STAGES) * BK, rows_valid, cols_valid, Ac, Bc);
            weave_half<2>();
            __builtin_amdgcn_sched_barrier(0);
        };
        // Whole rounds of STAGES slices, free of conditionals, then the rest.
        int s0 = s_begin;
        for (; s0 + STAGES <= s_end; s0 += STAGES) {
#pragma unroll
            for (int j = 0; j < STAGES; ++j)
                slice(s0 + j, Ast[j], Bst[j], Ast[(j + 1) % STAGES], Bst[(j + 1) % STAGES]);
        }
#pragma unroll
        for (int j = 0; j < STAGES - 1; ++j)
            if (s0 + j < s_end)
                slice(s0 + j, Ast[j], Bst[j], Ast[(j + 1) % STAGES], Bst[(j + 1) % STAGES]);
        // The zero-filling loads issued for slices past the end must land before
        // the workgroup's LDS can be handed to another workgroup.
        ring_barrier<0>();

    }

    __device__ __forceinline__ void store(const Args& a, const f32x16 (&acc)[BI][BJ]) const {
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = wm * WM + bi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    const int j = wn * WN + bj * 32 + c;
                    if (i < rows_valid && j < cols_valid)
                        store_out(a, (int64_t)m0 + i, (int64_t)n0 + j, acc[bi][bj][r]);
                }
    }
};

template <int BM, int BN, int WM, int WN, int BK, int STAGES, int WPE, bool VEC, bool FULL,
          bool TA = false, bool TB = false>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void k_mfma_pipe(Args a, int tiles_m, int tiles_n, int xcd_remap) {
    using Core = PipeCore<BM, BN, WM, WN, BK, STAGES, VEC, FULL, TA, TB>;
    // One LDS object per stage, so that the compiler can tell the stage being
    // filled from the stages being read (unused stages are dropped).
    __shared__ __attribute__((aligned(16))) float As0[Core::LDS_A];
    __shared__ __attribute__((aligned(16))) float Bs0[Core::LDS_B];
    __shared__ __attribute__((aligned(16))) float As1[Core::LDS_A];
    __shared__ __attribute__((aligned(16))) float Bs1[Core::LDS_B];
    __shared__ __attribute__((aligned(16))) float As2[STAGES > 2 ? Core::LDS_A : 4];
    __shared__ __attribute__((aligned(16))) float Bs2[STAGES > 2 ? Core::LDS_B : 4];
    __shared__ __attribute__((aligned(16))) float As3[STAGES > 3 ? Core::LDS_A : 4];
    __shared__ __attribute__((aligned(16))) float Bs3[STAGES > 3 ? Core::LDS_B : 4];
    float* const Ast[4] = {As0, As1, As2, As3};
    float* const Bst[4] = {Bs0, Bs1, Bs2, Bs3};

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, M128_GROUP_M, xcd_remap != 0, tm, tn);
    const Core core(a, tm, tn);
    f32x16 acc[Core::BI][Core::BJ];
    Core::zero(acc);
    core.mainloop(a, 0, (a.K + BK - 1) / BK, Ast, Bst, acc);
    core.store(a, acc);
}

// Stream-K form of k_mfma_pipe (SkPlan in common.hpp): workgroups below
// p.dp_tiles compute whole tiles; the others their runs of slices, a run
// covering a whole tile writing C, the others their partial tiles (summed by
// k_sk_fixup).
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int WPE, bool VEC, bool FULL,
          bool TA = false, bool TB = false>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void k_mfma_pipe_sk(Args a, int tiles_m, int tiles_n, int xcd_remap, SkPlan p) {
    using Core = PipeCore<BM, BN, WM, WN, BK, STAGES, VEC, FULL, TA, TB>;
    using Io = PartialIo<Core::BI, Core::BJ, Core::NT>;
    __shared__ __attribute__((aligned(16))) float As0[Core::LDS_A];
    __shared__ __attribute__((aligned(16))) float Bs0[Core::LDS_B];
    __shared__ __attribute__((aligned(16))) float As1[Core::LDS_A];
    __shared__ __attribute__((aligned(16))) float Bs1[Core::LDS_B];
    __shared__ __attribute__((aligned(16))) float As2[STAGES > 2 ? Core::LDS_A : 4];
    __shared__ __attribute__((aligned(16))) float Bs2[STAGES > 2 ? Core::LDS_B : 4];
    __shared__ __attribute__((aligned(16))) float As3[STAGES > 3 ? Core::LDS_A : 4];
    __shared__ __attribute__((aligned(16))) float Bs3[STAGES > 3 ? Core::LDS_B : 4];
    float* const Ast[4] = {As0, As1, As2, As3};
    float* const Bst[4] = {Bs0, Bs1, Bs2, Bs3};

    const int b = blockIdx.x;
    f32x16 acc[Core::BI][Core::BJ];
    int tm, tn;
    if (b < p.dp_tiles) {
        tile_of_first(b, p.dp_tiles, tiles_m, tiles_n, M128_GROUP_M, xcd_remap != 0, tm, tn);
        const Core core(a, tm, tn);
        Core::zero(acc);
        core.mainloop(a, 0, p.slices, Ast, Bst, acc);
        core.store(a, acc);
        return;
    }
    const int j = b - p.dp_tiles;
    const int U = p.sk_tiles * p.slices;
    int u = j * p.upw;
    const int u_end = (u + p.upw) < U ? (u + p.upw) : U;
    while (u < u_end) {
        const int st = u / p.slices;
        const int s0 = u - st * p.slices;
        const int s1 = (s0 + (u_end - u)) < p.slices ? (s0 + (u_end - u)) : p.slices;
        tile_of_first(p.dp_tiles + st, p.dp_tiles, tiles_m, tiles_n, M128_GROUP_M,
                      xcd_remap != 0, tm, tn);
        // The lane's fragment and epilogue offsets derive from its thread
        // index; hidden from the compiler here, they are recomputed per run
        // instead of being hoisted out of the loop (and spilled).
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const Core core(a, tm, tn, tid);
        Core::zero(acc);
        core.mainloop(a, s0, s1, Ast, Bst, acc);
        if (s0 == 0 && s1 == p.slices)
            core.store(a, acc);
        else
            Io::put(p.partials + (size_t)sk_slot(p, j, st) * BM * BN, core.t, acc);
        u += s1 - s0;
    }
}

// One workgroup per split tile: the sum of its pieces in K order, then the
// epilogue. A tile covered by a single run was written by that run.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
void k_sk_fixup(Args a, int tiles_m, int tiles_n, int xcd_remap, SkPlan p) {
    using Core = PipeCore<BM, BN, WM, WN, 16, 2, true, false, false, false>;
    using Io = PartialIo<Core::BI, Core::BJ, Core::NT>;
    const int st = blockIdx.x;
    const int j0 = st * p.slices / p.upw, j1 = (st * p.slices + p.slices - 1) / p.upw;
    if (j0 == j1) return;
    int tm, tn;
    tile_of_first(p.dp_tiles + st, p.dp_tiles, tiles_m, tiles_n, M128_GROUP_M, xcd_remap != 0,
                  tm, tn);
    const Core core(a, tm, tn);
    f32x16 acc[Core::BI][Core::BJ];
    constexpr size_t TILE = (size_t)BM * BN;
    Io::template gather<true>(p.partials + (size_t)sk_slot(p, j0, st) * TILE, core.t, acc);
    for (int jj = j0 + 1; jj <= j1; ++jj)
        Io::template gather<false>(p.partials + (size_t)sk_slot(p, jj, st) * TILE, core.t, acc);
    core.store(a, acc);
}

// ===========================================================================
// mfma_64x128_kg4: a 64x128 tile computed by 16 waves in four K-groups of
// four (each wave 32x64). Group g multiplies the slices
// g, g+4, g+8, ... from its own two LDS stages, so a compute unit holds 16
// waves of one tile instead of 4, and a shape with fewer tiles than compute
// units (the odd 1000x1531x777 has 192) still keeps four waves on every
// SIMD of the units it uses. The pages split K across blocks with a
// workspace ("Optimizing Matrix Multiply on CUDA, Part 2", "Selecting Among
// Three Kernels"); here the split stays inside the workgroup: the four
// partial tiles are summed through LDS in the fixed order g = 0, 1, 2, 3, so
// the result does not depend on timing. One workgroup per compute unit
// (96 KB of LDS).
// ===========================================================================
template <int BM, int BN, int WM, int WN, int BK, bool VEC, bool TA = false, bool TB = false>
__global__ __launch_bounds__(4 * (BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu((BM / WM) * (BN / WN), (BM / WM) * (BN / WN))))
void k_mfma_kgroup(Args a, int tiles_m, int tiles_n, int xcd_remap) {
    constexpr int KG = 4;
    constexpr int GT = (BM / WM) * (BN / WN) * 64;  // threads per K-group
    constexpr int WAVES_N = BN / WN;
    constexpr int BI = WM / 32, BJ = WN / 32;
    constexpr int PER_LANE = BI * BJ * 16;  // accumulators per lane
    using Dma = TileFillDma<BM, BN, BK, GT, VEC, TA, TB>;
    constexpr int BNP = Dma::BNP;
    // Stage objects, one per stage (so that the fill of one stage is never
    // taken for a write to the stage being read), each holding all groups.
    __shared__ __attribute__((aligned(16))) float As0[KG * BM * BK];
    __shared__ __attribute__((aligned(16))) float Bs0[KG * BK * BNP];
    __shared__ __attribute__((aligned(16))) float As1[KG * BM * BK];
    __shared__ __attribute__((aligned(16))) float Bs1[KG * BK * BNP];
    static_assert(KG == 4, "four K-groups");

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, M128_GROUP_M, xcd_remap != 0, tm, tn);
    const int m0 = __builtin_amdgcn_readfirstlane(tm * BM);
    const int n0 = __builtin_amdgcn_readfirstlane(tn * BN);
    const int rows_valid = (a.M - m0) < BM ? (a.M - m0) : BM;
    const int cols_valid = (a.N - n0) < BN ? (a.N - n0) : BN;
    const int t = threadIdx.x, lane = t & 63;
    const int g = __builtin_amdgcn_readfirstlane(t / GT), tl = t % GT, wl = tl >> 6;
    const int wm = wl / WAVES_N, wn = wl % WAVES_N;
    const int h = lane >> 5, c = lane & 31;

    f32x16 acc[BI][BJ];
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // This group's part of a stage starts at g * BM * BK (A) and
    // g * BK * BNP (B).
    const SubstepMma<BM, BNP, WM, WN, BK, TA, TB> mma(wm, wn, h, c, g * BM * BK, g * BK * BNP);
    auto compute = [&](const float* Ac, const float* Bc) { mma(Ac, Bc, acc); };

    // Step i: group g multiplies slice i*KG + g from the current stage while
    // its loads of slice (i+1)*KG + g fill the other one; one workgroup
    // barrier per step (it also waits for each wave's loads).
    const int nslices = (a.K + BK - 1) / BK;
    const int nsteps = (nslices + KG - 1) / KG;
    const Dma dma;
    auto step = [&](int i, float* Acur, float* Bcur, float* Anext, float* Bnext) {
        const int s = i * KG + g;
        if (s + KG < nslices)
            dma.issue(a, tl, m0, n0, (s + KG) * BK, rows_valid, cols_valid, Anext + g * BM * BK,
                      Bnext + g * BK * BNP);
        if (s < nslices) compute(Acur, Bcur);
        __syncthreads();
    };
    if (g < nslices)
        dma.issue(a, tl, m0, n0, g * BK, rows_valid, cols_valid, As0 + g * BM * BK,
                  Bs0 + g * BK * BNP);
    __syncthreads();
    for (int i = 0; i < nsteps; i += 2) {
        step(i, As0, Bs0, As1, Bs1);
        if (i + 1 < nsteps) step(i + 1, As1, Bs1, As0, Bs0);
    }

    // Fixed-order reduction of the four partial tiles (the last step's
    // barrier has retired every read of the stages).
    // Two-level tree in a fixed order, (p0 + p2) + (p1 + p3), through the
    // stages: each wave holds at most one partial tile besides its own. The
    // accumulators of a lane travel as 16-byte vectors; vector q of thread tl
    // goes to lo[(q*GT + tl)*4] for q < Q/2 and to hi[((q - Q/2)*GT + tl)*4]
    // above, so a wave's accesses are consecutive. Slot 0 is stage 0 and slot
    // 1 stage 1: each half of a slot is its B part when a whole partial tile
    // fits in it, else the A part and the B part.
    constexpr int Q = PER_LANE / 4;
    constexpr bool IN_B = KG * BK * BNP >= PER_LANE * GT;
    static_assert(IN_B || (KG * BK * BNP >= PER_LANE / 2 * GT && KG * BM * BK >= PER_LANE / 2 * GT),
                  "a partial tile must fit one LDS stage");
    auto slot = [&](int j, float*& lo, float*& hi) {
        float* A = j == 0 ? As0 : As1;
        float* B = j == 0 ? Bs0 : Bs1;
        lo = B + tl * 4;
        hi = (IN_B ? B + Q / 2 * GT * 4 : A) + tl * 4;
    };
    auto put = [&](int j) {
        float *lo, *hi;
        slot(j, lo, hi);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int bi = q / (4 * BJ), bj = (q / 4) % BJ, r0 = (q % 4) * 4;
            *(f32x4*)(q < Q / 2 ? lo + q * GT * 4 : hi + (q - Q / 2) * GT * 4) =
                f32x4{acc[bi][bj][r0], acc[bi][bj][r0 + 1], acc[bi][bj][r0 + 2], acc[bi][bj][r0 + 3]};
        }
    };
    auto add = [&](int j) {
        float *lo, *hi;
        slot(j, lo, hi);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int bi = q / (4 * BJ), bj = (q / 4) % BJ, r0 = (q % 4) * 4;
            const f32x4 v = *(const f32x4*)(q < Q / 2 ? lo + q * GT * 4 : hi + (q - Q / 2) * GT * 4);
            acc[bi][bj][r0] += v.x;
            acc[bi][bj][r0 + 1] += v.y;
            acc[bi][bj][r0 + 2] += v.z;
            acc[bi][bj][r0 + 3] += v.w;
            // After each 32x32 block: the block's sums must exist before
            // later loads issue, or the compiler loads the whole partial
            // tile first and spills registers.
            if (q % 4 == 3) asm volatile("" : "+v"(acc[bi][bj])::"memory");
        }
    };
    if (g == 2) put(0);
    if (g == 3) put(1);
    __syncthreads();
    if (g == 0) add(0);
    if (g == 1) add(1);
    __syncthreads();
    if (g == 1) put(0);
    __syncthreads();
    if (g != 0) return;
    add(0);

#pragma unroll
    for (int bi = 0; bi < BI; ++bi)
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = wm * WM + bi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const int j = wn * WN + bj * 32 + c;
                if (i < rows_valid && j < cols_valid)
                    store_out(a, (int64_t)m0 + i, (int64_t)n0 + j, acc[bi][bj][r]);
            }
}

// Host-side limits shared by the tiled MFMA kernels: per-slice buffer extents
// must stay below 2^31 bytes. A slice of A spans BM rows of BK (BK rows of
// BM when A is stored transposed); one of B spans BK rows of BN (BN rows of
// BK when transposed).
static bool extents_ok(const Args& a, int BM, int BN, int BK) {
    const int64_t ea = a.ta ? ((int64_t)(BK - 1) * a.lda + BM) * 4 : ((int64_t)(BM - 1) * a.lda + BK) * 4;
    const int64_t eb = a.tb ? ((int64_t)(BN - 1) * a.ldb + BK) * 4 : ((int64_t)(BK - 1) * a.ldb + BN) * 4;
    return ea < (int64_t)OOB && eb < (int64_t)OOB;
}

bool vec_ok(const Args& a) {
    const int ca = a.ta ? a.M : a.K, cb = a.tb ? a.K : a.N;
    return !((ca & 3) || (cb & 3) || (a.lda & 3) || (a.ldb & 3) || !aligned16(a.A) ||
             !aligned16(a.B));
}

// Calls f(std::integral_constant<bool, ta>, std::integral_constant<bool, tb>)
// with the call's transposition flags as compile-time constants.
template <class F>
static hipError_t with_trans(const Args& a, F&& f) {
    using T = std::true_type;
    using N = std::false_type;
    if (a.ta) return a.tb ? f(T{}, T{}) : f(T{}, N{});
    return a.tb ? f(N{}, T{}) : f(N{}, N{});
}

// mfma_256x256 tile parameters: the pipelined kernel with a 256x256 block
// tile, 16 waves of 64x64 (four per SIMD, all of one workgroup), one
// workgroup per compute unit (2 x 32 KiB LDS stages). With every wave of a
// compute unit in one workgroup there is no staggered finish between
// workgroups sharing a SIMD, and the A and B panels are read from L2 half as
// often as with 128x128 tiles.
#ifndef SGEMM_M256_BM
#define SGEMM_M256_BM 256
#endif
#ifndef SGEMM_M256_BN
#define SGEMM_M256_BN 256
#endif
#ifndef SGEMM_M256_WM
#define SGEMM_M256_WM 64
#endif
#ifndef SGEMM_M256_WN
#define SGEMM_M256_WN 64
#endif
#ifndef SGEMM_M256_WPE
#define SGEMM_M256_WPE 4
#endif
#ifndef SGEMM_M256_STAGES
#define SGEMM_M256_STAGES 2
#endif
#ifndef SGEMM_M256_BK
#define SGEMM_M256_BK 16
#endif

// An instance of the pipelined kernel (k_mfma_pipe, and k_mfma_pipe_sk for
// stream-K): block tile, wave tile, K slice, LDS stages and occupancy
// target. Per call it picks the FULL form (tile grid and K slices exactly
// cover the problem: no range masks) or the masked one, and the 16-byte or
// 4-byte fill (vec_ok). The 4-byte-fill form keeps more loads in flight per
// lane; it targets 3 waves per SIMD, or as many as one workgroup puts on
// each SIMD if that is more, since it would spill at 4.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int WPE>
struct PipeInstance {
    static constexpr int NT = (BM / WM) * (BN / WN) * 64;
    static constexpr int kBM = BM, kBN = BN, kBK = BK;
    static constexpr int WPE4 = NT / 256 > 3 ? NT / 256 : 3;

    static const void* kernel() {
        return (const void*)k_mfma_pipe<BM, BN, WM, WN, BK, STAGES, WPE, true, false>;
    }
    static const void* sk_kernel() {
        return (const void*)k_mfma_pipe_sk<BM, BN, WM, WN, BK, STAGES, WPE, true, false>;
    }
    static int check(const Args& a) {
        if (!extents_ok(a, BM, BN, BK)) return SGEMM_F32_ERR_TOO_LARGE;
        const int64_t tiles = cdiv(a.M, BM) * cdiv(a.N, BN);
        return tiles <= max_workgroups(NT) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
    }
    // f(VEC, FULL, TA, TB), each a std::integral_constant<bool>.
    template <class F>
    static hipError_t forms(const Args& a, F&& f) {
        using T = std::true_type;
        using N = std::false_type;
        const bool vec = vec_ok(a);
        const bool full = a.M % BM == 0 && a.N % BN == 0 && a.K % BK == 0;
        return with_trans(a, [&](auto ta, auto tb) {
            if (vec && full) return f(T{}, T{}, ta, tb);
            if (vec) return f(T{}, N{}, ta, tb);
            return f(N{}, N{}, ta, tb);
        });
    }
    static hipError_t launch(const Args& a, hipStream_t s) {
        const int tm = (int)cdiv(a.M, BM), tn = (int)cdiv(a.N, BN);
        const dim3 grid((unsigned)((int64_t)tm * tn)), block(NT);
        return forms(a, [&](auto vec, auto full, auto ta, auto tb) {
            constexpr bool V = decltype(vec)::value, F = decltype(full)::value;
            hipLaunchKernelGGL((k_mfma_pipe<BM, BN, WM, WN, BK, STAGES, V ? WPE : WPE4, V, F,
                                            decltype(ta)::value, decltype(tb)::value>),
                               grid, block, 0, s, a, tm, tn, xcd_remap_enabled());
            return hipGetLastError();
        });
    }

    // Stream-K: one workgroup per whole tile of the first rounds, then the
    // stream-K workgroups (sk_split), then k_sk_fixup on the same stream.
    static SkSplit split(const Args& a, int cus) {
        return sk_split(cdiv(a.M, BM) * cdiv(a.N, BN), cdiv(a.K, BK), cus);
    }
    static size_t ws_size(const Args& a, int cus) { return sk_workspace_bytes(split(a, cus), BM, BN); }
    static hipError_t launch_ws(const Args& a, void* ws, size_t ws_bytes, int cus, hipStream_t s) {
        const SkSplit sp = split(a, cus);
        if (!sp.split()) return launch(a, s);
        if (ws == nullptr || ws_bytes < sk_workspace_bytes(sp, BM, BN)) return hipErrorInvalidValue;
        SkPlan p;
        p.dp_tiles = (int)sp.dp_tiles;
        p.sk_tiles = (int)sp.sk_tiles;
        p.sk_wgs = (int)sp.sk_wgs;
        p.upw = (int)sp.upw;
        p.slices = (int)sp.slices;
        p.partials = (float*)ws;
        const int tm = (int)cdiv(a.M, BM), tn = (int)cdiv(a.N, BN);
        const dim3 grid((unsigned)(p.dp_tiles + p.sk_wgs)), block(NT);
        const hipError_t e = forms(a, [&](auto vec, auto full, auto ta, auto tb) {
            constexpr bool V = decltype(vec)::value, F = decltype(full)::value;
            hipLaunchKernelGGL((k_mfma_pipe_sk<BM, BN, WM, WN, BK, STAGES, V ? WPE : WPE4, V, F,
                                               decltype(ta)::value, decltype(tb)::value>),
                               grid, block, 0, s, a, tm, tn, xcd_remap_enabled(), p);
            return hipGetLastError();
        });
        // Runs as long as a tile (upw == slices) cover whole tiles only.
        if (e != hipSuccess || p.upw == p.slices) return e;
        hipLaunchKernelGGL((k_sk_fixup<BM, BN, WM, WN>), dim3((unsigned)p.sk_tiles), block, 0, s, a,
                           tm, tn, xcd_remap_enabled(), p);
        return hipGetLastError();
    }
};

using Pipe256 = PipeInstance<SGEMM_M256_BM, SGEMM_M256_BN, SGEMM_M256_WM, SGEMM_M256_WN,
                             SGEMM_M256_BK, SGEMM_M256_STAGES, SGEMM_M256_WPE>;
using Pipe128 = PipeInstance<M128_BM, M128_BN, M128_WM, M128_WN, M128_BK, 2,
                             SGEMM_M128_WAVES_PER_EU>;
// Two 24 KiB LDS stages per 4-wave workgroup: three workgroups per compute
// unit, so three waves per SIMD.
using Pipe64x128 =
    PipeInstance<64, 128, SGEMM_M64x128_WM, SGEMM_M64x128_WN, SGEMM_M64x128_BK, 2, 3>;

Variant kMfma256 = {"mfma_256x256", Pipe256::check, Pipe256::launch, Pipe256::kernel(),
                    Pipe256::NT, true, nullptr, nullptr, Pipe256::kBM, Pipe256::kBN, Pipe256::kBK};
Variant kMfma128 = {"mfma_128x128", Pipe128::check, Pipe128::launch, Pipe128::kernel(),
                    Pipe128::NT, true, nullptr, nullptr, Pipe128::kBM, Pipe128::kBN, Pipe128::kBK};
// 64x128: twice the tiles of mfma_128x128 for medium shapes (e.g. 3072^3,
// whose 576 tiles of 128x128 leave the second round of workgroups a third
// full).
Variant kMfma64x128 = {"mfma_64x128", Pipe64x128::check, Pipe64x128::launch,
                       Pipe64x128::kernel(), Pipe64x128::NT, true, nullptr, nullptr,
                       Pipe64x128::kBM, Pipe64x128::kBN, Pipe64x128::kBK};
// Stream-K forms (they need a workspace: sgemm_f32_ws).
Variant kMfma256Sk = {"mfma_256x256_sk", Pipe256::check, nullptr, Pipe256::sk_kernel(),
                      Pipe256::NT, true, Pipe256::ws_size, Pipe256::launch_ws,
                      Pipe256::kBM, Pipe256::kBN, Pipe256::kBK};
Variant kMfma128Sk = {"mfma_128x128_sk", Pipe128::check, nullptr, Pipe128::sk_kernel(),
                      Pipe128::NT, true, Pipe128::ws_size, Pipe128::launch_ws,
                      Pipe128::kBM, Pipe128::kBN, Pipe128::kBK};
Variant kMfma64x128Sk = {"mfma_64x128_sk", Pipe64x128::check, nullptr, Pipe64x128::sk_kernel(),
                         Pipe64x128::NT, true, Pipe64x128::ws_size, Pipe64x128::launch_ws,
                         Pipe64x128::kBM, Pipe64x128::kBN, Pipe64x128::kBK};

template <int BM, int BN, int WM, int WN, int BK = 16>
struct KgroupInstance {
    static constexpr int NT = 4 * (BM / WM) * (BN / WN) * 64;
    static constexpr int kBM = BM, kBN = BN, kBK = BK;
    static int check(const Args& a) {
        if (!extents_ok(a, BM, BN, BK)) return SGEMM_F32_ERR_TOO_LARGE;
        const int64_t tiles = cdiv(a.M, BM) * cdiv(a.N, BN);
        return tiles <= max_workgroups(NT) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
    }
    static hipError_t launch(const Args& a, hipStream_t s) {
        const int tm = (int)cdiv(a.M, BM), tn = (int)cdiv(a.N, BN);
        const dim3 grid((unsigned)((int64_t)tm * tn)), block(NT);
        const bool vec = vec_ok(a);
        return with_trans(a, [&](auto ta, auto tb) {
            constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
            if (vec)
                hipLaunchKernelGGL((k_mfma_kgroup<BM, BN, WM, WN, BK, true, TA, TB>), grid, block, 0, s,
                                   a, tm, tn, xcd_remap_enabled());
            else
                hipLaunchKernelGGL((k_mfma_kgroup<BM, BN, WM, WN, BK, false, TA, TB>), grid, block, 0,
                                   s, a, tm, tn, xcd_remap_enabled());
            return hipGetLastError();
        });
    }
    static const void* kernel() { return (const void*)k_mfma_kgroup<BM, BN, WM, WN, BK, true>; }
};

// 64x128 tile, 4 groups of 4 waves of 32x64 (16 waves, 96 KB LDS).
using Kg128 = KgroupInstance<64, 128, 32, 64>;
Variant kMfmaKgroup = {"mfma_64x128_kg4", Kg128::check, Kg128::launch, Kg128::kernel(), Kg128::NT,
                       true, nullptr, nullptr, Kg128::kBM, Kg128::kBN, Kg128::kBK};
// 64x96 tile, 4 groups of 3 waves of 64x32 (12 waves, 80 KB LDS): the odd
// 1000x1531 output is exactly 256 such tiles.
#ifndef SGEMM_KG96_BK
#define SGEMM_KG96_BK 16
#endif
using Kg96 = KgroupInstance<64, 96, 64, 32, SGEMM_KG96_BK>;
Variant kMfmaKgroup96 = {"mfma_64x96_kg4", Kg96::check, Kg96::launch, Kg96::kernel(), Kg96::NT,
                         true, nullptr, nullptr, Kg96::kBM, Kg96::kBN, Kg96::kBK};
// 128x128 tile, 4 groups of 4 waves of 64x64 (16 waves, 128 KB LDS): one
// tile per compute unit with four waves per SIMD, for shapes with at most
// about one 128x128 tile per compute unit and long K.
using Kg128x128 = KgroupInstance<128, 128, 64, 64>;
Variant kMfmaKgroup128 = {"mfma_128x128_kg4", Kg128x128::check, Kg128x128::launch,
                          Kg128x128::kernel(), Kg128x128::NT, true, nullptr, nullptr,
                          Kg128x128::kBM, Kg128x128::kBN, Kg128x128::kBK};

// ===========================================================================
// mfma_64: 64x64 block tile, BK = 16, 4 waves in 2x2, each wave 32x32 = 2x2
// blocks of 16x16 accumulated with v_mfma_f32_16x16x4_f32. Four times as many
// tiles as mfma_128 for shapes whose 128x128 grid leaves compute units idle.
// ===========================================================================
constexpr int M64_BM = 64, M64_BN = 64, M64_BK = 16, M64_GROUP_M = 8;

template <bool VEC>
__global__ __launch_bounds__(256) void k_mfma64(Args a, int tiles_m, int tiles_n, int xcd_remap) {
    constexpr int BM = M64_BM, BN = M64_BN, BK = M64_BK;
    using Fill = TileFill<BM, BN, BK, 256, VEC>;
    constexpr int BNP = Fill::BNP;
    __shared__ __attribute__((aligned(16))) float As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * BNP];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, M64_GROUP_M, xcd_remap != 0, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_valid = (a.M - m0) < BM ? (a.M - m0) : BM;
    const int cols_valid = (a.N - n0) < BN ? (a.N - n0) : BN;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int g = lane >> 4, c = lane & 15;

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    int aoff[2], boff[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
        const int row = wm * 32 + bi * 16 + c;
        aoff[bi] = row * BK + ((g ^ swz16(row)) << 2);
    }
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) boff[bj] = (4 * g) * BNP + wn * 32 + bj * 16 + c;

    const int nslices = (a.K + BK - 1) / BK;
    Fill fill;
    fill.load(a, t, m0, n0, 0, rows_valid, cols_valid);
    fill.store(As[0], Bs[0], t);
    __syncthreads();

    for (int s = 0; s < nslices; ++s) {
        const int cur = s & 1;
        if (s + 1 < nslices) fill.load(a, t, m0, n0, (s + 1) * BK, rows_valid, cols_valid);
        const float* Ac = As[cur];
        const float* Bc = Bs[cur];
        f32x4 af[2];
        float bf[2][4];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) af[bi] = *(const f32x4*)&Ac[aoff[bi]];
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int k = 0; k < 4; ++k) bf[bj][k] = Bc[boff[bj] + k * BNP];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < 2; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[bi][k], bf[bj][k],
                                                                       acc[bi][bj], 0, 0, 0);
        if (s + 1 < nslices) fill.store(As[cur ^ 1], Bs[cur ^ 1], t);
        __syncthreads();
    }

#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = wm * 32 + bi * 16 + 4 * g + r;
                const int j = wn * 32 + bj * 16 + c;
                if (i < rows_valid && j < cols_valid)
                    store_out(a, (int64_t)m0 + i, (int64_t)n0 + j, acc[bi][bj][r]);
            }
}

static int check_mfma64(const Args& a) {
    if (!extents_ok(a, M64_BM, M64_BN, M64_BK)) return SGEMM_F32_ERR_TOO_LARGE;
    const int64_t tiles = cdiv(a.M, M64_BM) * cdiv(a.N, M64_BN);
    return tiles <= max_workgroups(256) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
}

static hipError_t launch_mfma64(const Args& a, hipStream_t s) {
    const int tm = (int)cdiv(a.M, M64_BM), tn = (int)cdiv(a.N, M64_BN);
    const dim3 grid((unsigned)((int64_t)tm * tn)), block(256);
    if (vec_ok(a))
        hipLaunchKernelGGL(k_mfma64<true>, grid, block, 0, s, a, tm, tn, xcd_remap_enabled());
    else
        hipLaunchKernelGGL(k_mfma64<false>, grid, block, 0, s, a, tm, tn, xcd_remap_enabled());
    return hipGetLastError();
}

Variant kMfma64 = {"mfma_64x64", check_mfma64, launch_mfma64, (const void*)k_mfma64<true>,
                   256, false, nullptr, nullptr, M64_BM, M64_BN, M64_BK};

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
// ===========================================================================
#ifndef SGEMM_DIRECT_TM
#define SGEMM_DIRECT_TM 32
#endif
#ifndef SGEMM_DIRECT_TN
#define SGEMM_DIRECT_TN 32
#endif
#ifndef SGEMM_DIRECT_KS
#define SGEMM_DIRECT_KS 4
#endif
constexpr int DR_TM = SGEMM_DIRECT_TM, DR_TN = SGEMM_DIRECT_TN, DR_KS = SGEMM_DIRECT_KS;
constexpr int DR_GROUP_M = 8;

template <int TM, int TN, bool VEC>
struct DirectFrag {
    static constexpr int BI = TM / 32, BJ = TN / 32;
    float a[BI][8];
    float b[BJ][8];

    // Step starting at k0: lane (h, c) reads A[m0 + 32*bi + c][k0 + 8h + 0..7]
    // and B[k0 + 8h + s][n0 + 32*bj + c]; everything outside the matrix reads 0.
    __device__ __forceinline__ void load(const Args& a_, int m0, int n0, int k0, int rows_valid,
                                         int cols_valid, int h, int c) {
        const int kk = (a_.K - k0) < 16 ? (a_.K - k0) : 16;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(
            a_.A + (int64_t)m0 * a_.lda + k0, (uint32_t)(((int64_t)(rows_valid - 1) * a_.lda + kk) * 4));
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(
            a_.B + (int64_t)k0 * a_.ldb + n0, (uint32_t)(((int64_t)(kk - 1) * a_.ldb + cols_valid) * 4));
#pragma unroll
        for (int bi = 0; bi < BI; ++bi) {
            const int row = 32 * bi + c;
            const bool rok = row < rows_valid;
            if (VEC) {
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
                    a[bi][s] = buf_load1(rA, rok && kq < kk ? (uint32_t)((row * (int)a_.lda + kq) * 4) : OOB);
                }
            }
        }
#pragma unroll
        for (int bj = 0; bj < BJ; ++bj) {
            const int col = 32 * bj + c;
            const bool cok = col < cols_valid;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int kr = 8 * h + s;
                b[bj][s] = buf_load1(rB, cok && kr < kk ? (uint32_t)((kr * (int)a_.ldb + col) * 4) : OOB);
            }
        }
    }
};

template <int TM, int TN, int KS, bool VEC>
__global__ __launch_bounds__(64 * KS) void k_mfma_direct(Args a, int tiles_m, int tiles_n,
                                                         int xcd_remap) {
    constexpr int BI = TM / 32, BJ = TN / 32, NB = BI * BJ;
    __shared__ float red[KS * NB * 16 * 64];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, DR_GROUP_M, xcd_remap != 0, tm, tn);
    const int m0 = tm * TM, n0 = tn * TN;
    const int rows_valid = (a.M - m0) < TM ? (a.M - m0) : TM;
    const int cols_valid = (a.N - n0) < TN ? (a.N - n0) : TN;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = lane >> 5, c = lane & 31;

    f32x16 acc[BI][BJ];
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nsteps = (a.K + 15) / 16;
    DirectFrag<TM, TN, VEC> cur, nxt;
    if (w < nsteps) cur.load(a, m0, n0, 16 * w, rows_valid, cols_valid, h, c);
    for (int j = w; j < nsteps; j += KS) {
        if (j + KS < nsteps) nxt.load(a, m0, n0, 16 * (j + KS), rows_valid, cols_valid, h, c);
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(cur.a[bi][s], cur.b[bj][s],
                                                                       acc[bi][bj], 0, 0, 0);
        cur = nxt;
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
    for (int blk = w; blk < NB; blk += KS) {
        const int bi = blk / BJ, bj = blk % BJ;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float v = red[((0 * NB + blk) * 16 + r) * 64 + lane];
#pragma unroll
            for (int ww = 1; ww < KS; ++ww) v += red[((ww * NB + blk) * 16 + r) * 64 + lane];
            const int i = bi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const int jj = bj * 32 + c;
            if (i < rows_valid && jj < cols_valid)
                store_out(a, (int64_t)m0 + i, (int64_t)n0 + jj, v);
        }
    }
}

static int check_direct(const Args& a) {
    const int64_t ea = ((int64_t)(DR_TM - 1) * a.lda + 16) * 4;
    const int64_t eb = ((int64_t)15 * a.ldb + DR_TN) * 4;
    if (ea >= (int64_t)OOB || eb >= (int64_t)OOB) return SGEMM_F32_ERR_TOO_LARGE;
    const int64_t tiles = cdiv(a.M, DR_TM) * cdiv(a.N, DR_TN);
    return tiles <= max_workgroups(64 * DR_KS) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
}

static hipError_t launch_direct(const Args& a, hipStream_t s) {
    const int tm = (int)cdiv(a.M, DR_TM), tn = (int)cdiv(a.N, DR_TN);
    const dim3 grid((unsigned)((int64_t)tm * tn)), block(64 * DR_KS);
    const bool vec = !((a.K & 3) || (a.lda & 3) || !aligned16(a.A));
    if (vec)
        hipLaunchKernelGGL((k_mfma_direct<DR_TM, DR_TN, DR_KS, true>), grid, block, 0, s, a, tm, tn,
                           xcd_remap_enabled());
    else
        hipLaunchKernelGGL((k_mfma_direct<DR_TM, DR_TN, DR_KS, false>), grid, block, 0, s, a, tm, tn,
                           xcd_remap_enabled());
    return hipGetLastError();
}

Variant kMfmaDirect = {"mfma_direct", check_direct, launch_direct,
                       (const void*)k_mfma_direct<DR_TM, DR_TN, DR_KS, true>, 64 * DR_KS};

// ===========================================================================
// mfma_skinny: for few rows (near-GEMV, e.g. 16 x 8192 x 8192, where B is
// read once and the shape is bound by HBM bandwidth). A workgroup owns a
// 16x32 tile of C and all of K; its 16 waves each take one contiguous 1/16 of
// K, so 16 independent streams of B loads are in flight per compute unit.
// Operands go straight from global memory into MFMA registers (no LDS tile):
// lane l of a wave reads row k = 4*(l/16) + s of its K run at column l%16 of
// each 16-column block, 64 contiguous bytes per quarter-wave, and a 16-byte
// run of 4 consecutive k of row l%16 of A. At the end the 16 partial tiles
// are summed in a fixed order through LDS (deterministic) and the epilogue
// writes C.
// ===========================================================================
constexpr int SK_BM = 16, SK_BN = 32, SK_WAVES = 16, SK_KU = 64;  // k per unrolled step

template <bool VEC>
__global__ __launch_bounds__(1024) void k_mfma_skinny(Args a, int tiles_n, int kchunk) {
    __shared__ float red[SK_WAVES][2][4][64];
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * SK_BM, n0 = tn * SK_BN;
    const int rows_valid = (a.M - m0) < SK_BM ? (a.M - m0) : SK_BM;
    const int cols_valid = (a.N - n0) < SK_BN ? (a.N - n0) : SK_BN;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const int kbeg = w * kchunk;
    const int kend = (a.K - kbeg) < kchunk ? a.K : kbeg + kchunk;

    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = kbeg; k0 < kend; k0 += SK_KU) {
        const int kk = (a.K - k0) < SK_KU ? (a.K - k0) : SK_KU;  // rows present in memory
        const int klim = kend - k0;                              // rows this wave owns
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(
            a.A + (int64_t)m0 * a.lda + k0, (uint32_t)(((int64_t)(rows_valid - 1) * a.lda + kk) * 4));
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(
            a.B + (int64_t)k0 * a.ldb + n0, (uint32_t)(((int64_t)(kk - 1) * a.ldb + cols_valid) * 4));
        f32x4 af[SK_KU / 16];
        float b0[SK_KU / 4], b1[SK_KU / 4];
#pragma unroll
        for (int u = 0; u < SK_KU / 16; ++u) {
            const int kq = 16 * u + 4 * g;  // this lane's 4 consecutive k
            if (VEC) {
                const bool ok = c < rows_valid && kq + 4 <= klim;
                af[u] = buf_load4(rA, ok ? (uint32_t)((c * (int)a.lda + kq) * 4) : OOB);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = c < rows_valid && kq + e < klim;
                    af[u][e] = buf_load1(rA, ok ? (uint32_t)((c * (int)a.lda + kq + e) * 4) : OOB);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kr = kq + e;
                const bool okr = kr < klim;
                const uint32_t base = (uint32_t)(kr * (int)a.ldb) * 4;
                b0[4 * u + e] = buf_load1(rB, okr && c < cols_valid ? base + c * 4 : OOB);
                b1[4 * u + e] = buf_load1(rB, okr && c + 16 < cols_valid ? base + (c + 16) * 4 : OOB);
            }
        }
#pragma unroll
        for (int u = 0; u < SK_KU / 16; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(af[u][e], b0[4 * u + e], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(af[u][e], b1[4 * u + e], acc1, 0, 0, 0);
            }
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) {
        red[w][0][r][lane] = acc0[r];
        red[w][1][r][lane] = acc1[r];
    }
    __syncthreads();
    if (threadIdx.x < SK_BM * SK_BN) {
        const int i = threadIdx.x / SK_BN, j = threadIdx.x % SK_BN;
        const int bj = j >> 4, src = (i >> 2) * 16 + (j & 15), r = i & 3;
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < SK_WAVES; ++ww) v += red[ww][bj][r][src];
        if (i < rows_valid && j < cols_valid) store_out(a, (int64_t)m0 + i, (int64_t)n0 + j, v);
    }
}

static int skinny_kchunk(const Args& a) {
    // Equal K runs per wave, each a multiple of 16.
    const int64_t per = cdiv(a.K, SK_WAVES);
    return (int)(cdiv(per, 16) * 16);
}

static int check_skinny(const Args& a) {
    const int64_t ea = ((int64_t)(SK_BM - 1) * a.lda + SK_KU) * 4;
    const int64_t eb = ((int64_t)(SK_KU - 1) * a.ldb + SK_BN) * 4;
    if (ea >= (int64_t)OOB || eb >= (int64_t)OOB) return SGEMM_F32_ERR_TOO_LARGE;
    const int64_t tiles = cdiv(a.M, SK_BM) * cdiv(a.N, SK_BN);
    return tiles <= max_workgroups(1024) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
}

static hipError_t launch_skinny(const Args& a, hipStream_t s) {
    const int tn = (int)cdiv(a.N, SK_BN);
    const dim3 grid((unsigned)(cdiv(a.M, SK_BM) * tn)), block(1024);
    const bool vec = !((a.K & 3) || (a.lda & 3) || !aligned16(a.A));
    if (vec)
        hipLaunchKernelGGL(k_mfma_skinny<true>, grid, block, 0, s, a, tn, skinny_kchunk(a));
    else
        hipLaunchKernelGGL(k_mfma_skinny<false>, grid, block, 0, s, a, tn, skinny_kchunk(a));
    return hipGetLastError();
}

Variant kMfmaSkinny = {"mfma_skinny", check_skinny, launch_skinny,
                             (const void*)k_mfma_skinny<true>, 1024};

}  // namespace sgemm
