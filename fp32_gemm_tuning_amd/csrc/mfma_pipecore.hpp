// The software-pipelined main loop of the tiled matrix-core kernels
// (PipeCore): a ring of LDS stages filled by buffer-to-LDS loads, fragment
// double buffering, the workgroup barrier between the last two parts of a
// slice, and fragment reads and fills woven between the MFMAs. Used by the
// pipelined kernel (mfma_pipe.hip) and by the K-group kernels with 16-byte
// fills (mfma_kgroup.hip).
#pragma once

#include "mfma_common.hpp"

namespace sgemm {

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
// FRONT, for parts of at most 8 MFMAs (wave tiles of one or two 32x32
// blocks, one or two waves per SIMD): the reads go out in pairs after each
// of the first two MFMAs, and the loads in pairs after the next three, so
// every read has at least six MFMAs to land instead of two. With few waves
// per SIMD no other wave covers a read that arrives late (interleaved A/B,
// bit-identical: 512x4096x4096 on the 64x128 tile 127.4 -> 123.8 us back
// to back, on the 64x64 tile 127.3 -> 124.2, 3072^3 411.3 -> 406.8, 2048^3
// 122.4 -> 121.5). The 16-MFMA parts of the 256x256 tile keep the pattern
// above (front-loaded there, the headline instance spills).
template <int LOADS, bool FRONT = false>
__device__ __forceinline__ void weave_half() {
    constexpr int MFMA = 0x008, VMEM_READ = 0x020, DS_READ = 0x100;
    if constexpr (FRONT) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(DS_READ, 2, 0);
        }
        if constexpr (LOADS > 0) {
#pragma unroll
            for (int l = 0; l < 3; ++l) {
                __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(VMEM_READ, 2, 0);
            }
        }
    } else if constexpr (LOADS == 0) {
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
//
// U16 (with VEC false and two stages): operands whose rows are not whole
// 16-byte chunks, filled with 16-byte loads into registers (OperandFillU).
// The prologue loads both stages' slices at once (two register sets); in the
// loop, the loads of slice s + 2, issued after slice s's barrier, are
// written into the stage slice s released just before slice s + 1's
// barrier: the same time for the loads to land as the buffer-to-LDS ring
// gives, with a quarter of the load instructions of the 4-byte fill.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, bool VEC, bool FULL, bool TA,
          bool TB, bool U16 = false>
struct PipeCore {
    static_assert(!U16 || (!VEC && !FULL && STAGES == 2), "the register fill serves a two-stage ring");
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
    // Front-loaded weave (weave_half) for parts of at most 8 MFMAs, with the
    // 16-byte fills: the 4-byte-fill forms of the 64x128 tile would spill.
    static constexpr bool FRONT = 4 * BI * BJ <= 8 && (VEC || U16);

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

    // Steps s_begin .. s_end - 1; step s multiplies K slice s * KSTRIDE + koff
    // (a K-group kernel gives each group every KSTRIDE-th slice). Slices at or
    // past the end of K load as zeros.
    // GUARD: s_math_end is s_end or s_end - 1 (a K-group whose slices ended
    // one step before the other groups'); the last step is then split off
    // and its fragment reads and MFMAs, which would multiply zeros, are
    // skipped when s_math_end < s_end.
    template <int KSTRIDE = 1, bool GUARD = false>
    __device__ __forceinline__ void mainloop(const Args& a, int s_begin, int s_end,
                                             float* const (&Ast)[4], float* const (&Bst)[4],
                                             f32x16 (&acc)[BI][BJ], int koff = 0,
                                             int s_math_end = 0) const {
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
        OperandFillU<BM, BK, NT, !TA> ua;
        OperandFillU<BN, BK, NT, TB> ub;
        if constexpr (U16) {
            ua.init(a.lda, m0, rows_valid, t);
            ub.init(a.ldb, n0, cols_valid, t);
        }
        bool pending = false;   // (U16) registers hold a slice to be written
        PartFrag<BI, BJ> f0, f1;
        // Prologue: fill every stage (stages past the last slice read zeros),
        // wait for slice 0, read its first half. Every slice below issues exactly
        // G loads per wave, whether or not its target slice exists, so the count
        // of loads issued after any given one is the same on every path.
        if constexpr (U16) {
            // Both prologue slices through registers, in flight together.
            OperandFillU<BM, BK, NT, !TA> ua1 = ua;
            OperandFillU<BN, BK, NT, TB> ub1 = ub;
            const int k0 = (s_begin * KSTRIDE + koff) * BK, k1 = ((s_begin + 1) * KSTRIDE + koff) * BK;
            ua.load(a.A, a.lda, m0, k0, a.K, rows_valid, t);
            ub.load(a.B, a.ldb, n0, k0, a.K, cols_valid, t);
            ua1.load(a.A, a.lda, m0, k1, a.K, rows_valid, t);
            ub1.load(a.B, a.ldb, n0, k1, a.K, cols_valid, t);
            ua.store(Ast[0], k0, t);
            ub.store(Bst[0], k0, t);
            ua1.store(Ast[1], k1, t);
            ub1.store(Bst[1], k1, t);
        } else {
#pragma unroll
            for (int j = 0; j < STAGES; ++j)
                dma.template issue<FULL>(a, t, m0, n0, ((s_begin + j) * KSTRIDE + koff) * BK, rows_valid,
                                         cols_valid, Ast[j], Bst[j]);
        }
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
        // The MFMAs of parts 0 .. P-2 of a slice from the current stage, with
        // the reads of parts 1 .. P-1 woven in.
        auto parts = [&](const float* Ac, const float* Bc) {
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
                weave_half<0, FRONT>();
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto slice = [&](int s, float* Ac, float* Bc, float* An, float* Bn) {
            parts(Ac, Bc);
            if constexpr (U16) {
                // Slice s + 1 into the stage slice s - 1 released (An).
                if (pending) {
                    const int k1 = ((s + 1) * KSTRIDE + koff) * BK;
                    ua.store(An, k1, t);
                    ub.store(Bn, k1, t);
                }
            }
            ring_barrier<(STAGES - 2) * G>();
            const int k2 = ((s + STAGES) * KSTRIDE + koff) * BK;
            auto issue = [&]() {
                if constexpr (U16) {
                    ua.load(a.A, a.lda, m0, k2, a.K, rows_valid, t);
                    ub.load(a.B, a.ldb, n0, k2, a.K, cols_valid, t);
                    pending = true;
                } else {
                    dma.template issue<FULL>(a, t, m0, n0, k2, rows_valid, cols_valid, Ac, Bc);
                }
            };
            read_part(f0, An, Bn, 0);   // past the last slice: read and unused
            mma_part(f1);
            issue();
            weave_half<U16 ? 0 : 2, FRONT>();
            __builtin_amdgcn_sched_barrier(0);
        };
        // GUARD: the last step, whose slice exists only for groups with
        // s_math_end == s_end; it loads nothing more.
        auto last_slice = [&](int s, const float* Ac, const float* Bc) {
            const bool cur = s < s_math_end;
            if (cur) parts(Ac, Bc);
            ring_barrier<(STAGES - 2) * G>();
            if (cur) mma_part(f1);
            __builtin_amdgcn_sched_barrier(0);
        };
        // Whole rounds of STAGES slices, free of conditionals, then the rest
        // (with GUARD, up to the last step, which follows on its own).
        const int s_stop = GUARD ? s_end - 1 : s_end;
        int s0 = s_begin;
        for (; s0 + STAGES <= s_stop; s0 += STAGES) {
#pragma unroll
            for (int j = 0; j < STAGES; ++j)
                slice(s0 + j, Ast[j], Bst[j], Ast[(j + 1) % STAGES], Bst[(j + 1) % STAGES]);
        }
#pragma unroll
        for (int j = 0; j < STAGES - 1; ++j)
            if (s0 + j < s_stop)
                slice(s0 + j, Ast[j], Bst[j], Ast[(j + 1) % STAGES], Bst[(j + 1) % STAGES]);
        if constexpr (GUARD) {
            if (s_end > s_begin) {
                const int j = (s_end - 1 - s_begin) % STAGES;
                last_slice(s_end - 1, Ast[j], Bst[j]);
            }
        }
        // The zero-filling loads issued for slices past the end must land before
        // the workgroup's LDS can be handed to another workgroup.
        ring_barrier<0>();

    }

    __device__ __forceinline__ void store(const Args& a, const f32x16 (&acc)[BI][BJ]) const {
        // The lane's output coordinates, recomputed from an opaque copy of
        // the thread index: derived before the main loop, the compiler kept
        // them live across it at four waves per SIMD and spilled them.
        int tt = t;
        asm volatile("" : "+v"(tt));
        const int lane = tt & 63, w = tt >> 6;
        const int wm_ = w / WAVES_N, wn_ = w % WAVES_N, h_ = lane >> 5, c_ = lane & 31;
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = wm_ * WM + bi * 32 + 8 * (r >> 2) + 4 * h_ + (r & 3);
                    const int j = wn_ * WN + bj * 32 + c_;
                    if (i < rows_valid && j < cols_valid)
                        store_out(a, (int64_t)m0 + i, (int64_t)n0 + j, acc[bi][bj][r]);
                }
    }
};

}  // namespace sgemm
