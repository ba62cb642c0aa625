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
//
// This header holds what the matrix-core kernel families share: the LDS fills
// (register-staged and buffer-to-LDS), the host-side limits, and the tile
// grouping of the tile mapping. The families live in mfma_pipe.hip (the
// pipelined kernel: mfma_256x256, mfma_128x128, mfma_64x128 and their
// stream-K forms), mfma_kgroup.hip (the K-group kernels) and mfma_small.hip
// (mfma_64x64, mfma_64x64_k4, mfma_direct, mfma_skinny).
#pragma once

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

// One operand's part of a K slice, filled through registers with 16-byte
// loads from addresses that need only be 4-byte aligned (gfx950 serves
// unaligned vector loads from global memory): for rows that are not whole
// 16-byte chunks (a leading dimension, contiguous extent or base address
// that is not a multiple of 4 floats), where the buffer-to-LDS fill would
// need one 4-byte load per element. The LDS layout and the lane of each
// chunk are those of OperandFill's 16-byte form (the lane inverts the A
// swizzle, so a wave's LDS writes are 1 KiB contiguous).
//
// No 16-byte load reaches past the operand's valid elements. A chunk whose
// four elements are all valid loads them directly. A chunk that straddles
// the end of the valid range along its contiguous dimension (the K tail for a
// k-contiguous operand, the edge of M or N for a row-contiguous one), with
// v < 4 valid elements, loads the last four valid elements instead, starting
// 4 - v elements earlier, and its lanes shift them down in registers and zero
// the rest. Chunks with no valid element read as zero: through the
// out-of-range offset, or, for the k rows of a row-contiguous operand past
// the K tail, because the slice's resource ends before them.
//
// Per-lane offsets are fixed for a tile (init): a whole slice of a
// k-contiguous operand only moves the resource base by the slice's k0, and
// every slice of a row-contiguous one moves it by k0 rows. Only the K-tail
// slice of a k-contiguous operand computes its offsets per lane. The host
// keeps the contiguous extent of the whole operand (K, or M/N) at least 4, so
// a shifted start never precedes the row, and (rows - 1) * ld + extent below
// 2^31 bytes.
template <int ROWS, int BK, int NT, bool KCONTIG>
struct OperandFillU {
    static constexpr int W = NT / 64;
    static constexpr int TOTAL = ROWS * BK / 256;       // pieces of 64 chunks
    static_assert(TOTAL * 256 == ROWS * BK, "tile/instruction mismatch");
    static constexpr int INSTR = (TOTAL + W - 1) / W;   // per wave per slice, at most
    static constexpr bool EVEN = TOTAL % W == 0;
    static constexpr int CPR = BK / 4;                  // 16-byte chunks per k-contiguous row
    static constexpr int CPK = ROWS / 4;                // chunks per k row of a row-contiguous one
    static_assert(ROWS % 4 == 0, "whole chunks per k row");

    f32x4 v[INSTR];
    uint32_t off[INSTR];   // byte offsets of a whole slice from its resource base (OOB: zero)
    int sh[INSTR];         // (row-contiguous) shift of a straddling chunk, else 0
    int kk;                // valid k of the slice in flight
    int edge;              // (row-contiguous) some chunk straddles the edge of M or N

    // Offsets from the resource base of a slice: row `line` of the tile at
    // k0 (k-contiguous), or k row `line` of the slice at column 0
    // (row-contiguous).
    __device__ __forceinline__ void init(int64_t ld, int r0, int rows_valid, int t) {
        const int ldi = (int)ld;
        const int w = t >> 6, lane = t & 63;
        edge = KCONTIG ? 0 : (rows_valid & 3);
#pragma unroll
        for (int p = 0; p < INSTR; ++p) {
            const int slot = (w + W * p) * 64 + lane;
            if (KCONTIG) {
                const int line = slot / CPR, q = (slot % CPR) ^ swz_chunk<BK>(line);
                off[p] = line < rows_valid ? (uint32_t)((line * ldi + 4 * q) * 4) : OOB;
                sh[p] = 0;
            } else {
                const int line = slot / CPK, c = r0 + 4 * (slot % CPK), cend = r0 + rows_valid;
                const bool straddle = c < cend && c + 4 > cend;
                off[p] = c < cend ? (uint32_t)((line * ldi + (straddle ? cend - 4 : c)) * 4) : OOB;
                sh[p] = straddle ? c + 4 - cend : 0;
            }
        }
    }

    // Global -> registers for the slice starting at k0 of rows r0 .. r0 +
    // rows_valid - 1 (X as stored: element (row, k) at X[row*ld + k] when
    // k-contiguous, else X[k*ld + row]).
    __device__ __forceinline__ void load(const float* X, int64_t ld, int r0, int k0, int K,
                                         int rows_valid, int t) {
        const int kr = K - k0;
        kk = __builtin_amdgcn_readfirstlane(kr <= 0 ? 0 : (kr < BK ? kr : BK));
        const int w = t >> 6, lane = t & 63;
        if (KCONTIG && kk > 0 && kk < BK) {
            // The K tail: per-lane range checks and shifted starts, from a
            // resource at column 0 of the tile's first row.
            const __amdgpu_buffer_rsrc_t r = make_rsrc(
                X + (int64_t)r0 * ld, (uint32_t)(((int64_t)(rows_valid - 1) * ld + k0 + kk) * 4));
            const int ldi = (int)ld, cend = k0 + kk;
#pragma unroll
            for (int p = 0; p < INSTR; ++p) {
                const int piece = w + W * p;
                if (!EVEN && piece >= TOTAL) break;
                const int slot = piece * 64 + lane;
                const int line = slot / CPR, c0 = k0 + 4 * ((slot % CPR) ^ swz_chunk<BK>(line));
                const bool ok = line < rows_valid && c0 < cend;
                const int cs = c0 + 4 <= cend ? c0 : cend - 4;
                v[p] = buf_load4(r, ok ? (uint32_t)((line * ldi + cs) * 4) : OOB);
            }
            return;
        }
        __amdgpu_buffer_rsrc_t r;
        if (KCONTIG)
            r = make_rsrc(X + (int64_t)r0 * ld + k0,
                          kk > 0 ? (uint32_t)(((int64_t)(rows_valid - 1) * ld + BK) * 4) : 0u);
        else
            r = make_rsrc(X + (int64_t)k0 * ld,
                          kk > 0 ? (uint32_t)(((int64_t)(kk - 1) * ld + r0 + rows_valid) * 4) : 0u);
#pragma unroll
        for (int p = 0; p < INSTR; ++p) {
            if (!EVEN && w + W * p >= TOTAL) break;
            v[p] = buf_load4(r, off[p]);
        }
    }

    // Registers -> LDS at dst_base (the operand's part of the stage), for the
    // slice `load` last fetched (k0 as given there).
    __device__ __forceinline__ void store(float* dst_base, int k0, int t) const {
        const int w = t >> 6, lane = t & 63;
#pragma unroll
        for (int p = 0; p < INSTR; ++p) {
            const int piece = w + W * p;
            if (!EVEN && piece >= TOTAL) break;
            const int slot = piece * 64 + lane;
            f32x4 x = v[p];
            int s = 0;
            if (KCONTIG) {
                if (kk & 3) {   // the K tail with a straddling chunk
                    const int c0 = k0 + 4 * ((slot % CPR) ^ swz_chunk<BK>(slot / CPR)), cend = k0 + kk;
                    s = (c0 < cend && c0 + 4 > cend) ? c0 + 4 - cend : 0;
                }
            } else if (edge) {
                s = sh[p];
            }
            if ((KCONTIG && (kk & 3)) || (!KCONTIG && edge)) {
                // Lanes of a straddling chunk hold the elements from its
                // shifted start; move element e + s to e and zero the rest.
                const float e0 = s == 0 ? x.x : s == 1 ? x.y : s == 2 ? x.z : x.w;
                const float e1 = s == 0 ? x.y : s == 1 ? x.z : s == 2 ? x.w : 0.0f;
                const float e2 = s == 0 ? x.z : s == 1 ? x.w : 0.0f;
                const float e3 = s == 0 ? x.w : 0.0f;
                x = f32x4{e0, e1, e2, e3};
            }
            *(f32x4*)(dst_base + slot * 4) = x;
        }
    }
};

// Host side of OperandFillU: the contiguous extent of each operand (K of A,
// N of B; M of a transposed A, K of a transposed B) is at least 4, and every
// offset of a slice's resource stays below 2^31 bytes.
static inline bool fillu_ok(const Args& a, int BM, int BN, int BK) {
    const int64_t ca = a.ta ? a.M : a.K, cb = a.tb ? a.K : a.N;
    if (ca < 4 || cb < 4) return false;
    const int64_t ea = a.ta ? ((int64_t)(BK - 1) * a.lda + a.M) * 4 : ((int64_t)(BM - 1) * a.lda + a.K) * 4;
    const int64_t eb = a.tb ? ((int64_t)(BN - 1) * a.ldb + a.K) * 4 : ((int64_t)(BK - 1) * a.ldb + a.N) * 4;
    return ea < (int64_t)OOB && eb < (int64_t)OOB;
}

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

// Tile-grouping band of the tile mapping (tile_of) for the tiled kernels.
#ifndef SGEMM_M128_GROUP_M
#define SGEMM_M128_GROUP_M 8
#endif
constexpr int M128_GROUP_M = SGEMM_M128_GROUP_M;

// Host-side limits shared by the tiled MFMA kernels: per-slice buffer extents
// must stay below 2^31 bytes. A slice of A spans BM rows of BK (BK rows of
// BM when A is stored transposed); one of B spans BK rows of BN (BN rows of
// BK when transposed).
static inline bool extents_ok(const Args& a, int BM, int BN, int BK) {
    const int64_t ea = a.ta ? ((int64_t)(BK - 1) * a.lda + BM) * 4 : ((int64_t)(BM - 1) * a.lda + BK) * 4;
    const int64_t eb = a.tb ? ((int64_t)(BN - 1) * a.ldb + BK) * 4 : ((int64_t)(BK - 1) * a.ldb + BN) * 4;
    return ea < (int64_t)OOB && eb < (int64_t)OOB;
}

// Calls f(std::integral_constant<bool, ta>, std::integral_constant<bool, tb>)
// with the call's transposition flags as compile-time constants.
template <class F>
static inline hipError_t with_trans(const Args& a, F&& f) {
    using T = std::true_type;
    using N = std::false_type;
    if (a.ta) return a.tb ? f(T{}, T{}) : f(T{}, N{});
    return a.tb ? f(N{}, T{}) : f(N{}, N{});
}

}  // namespace sgemm
