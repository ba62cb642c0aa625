// K-group FP32 matrix-core kernels (k_mfma_kgroup): mfma_64x128_kg4,
// mfma_64x96_kg4, mfma_96x64_kg4 and mfma_128x128_kg4, one tile per workgroup of four groups
// of waves that split the K slices and sum their partial tiles in a fixed
// order. Operand layouts and edge handling: mfma_common.hpp.
#include "mfma_pipecore.hpp"

namespace sgemm {

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
// How the K-group kernels fill a slice: buffer-to-LDS loads of 16 bytes
// (every operand row a whole number of 16-byte chunks), 16-byte loads
// through registers from 4-byte aligned rows (OperandFillU), or
// buffer-to-LDS loads of 4 bytes (any rows).
enum KgFill { KG_DMA4 = 0, KG_U16 = 1, KG_DMA16 = 2 };

template <int BM, int BN, int WM, int WN, int BK, int FILL, bool TA = false, bool TB = false>
__global__ __launch_bounds__(4 * (BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu((BM / WM) * (BN / WN), (BM / WM) * (BN / WN))))
void k_mfma_kgroup(Args a, int tiles_m, int tiles_n, int xcd_remap) {
    constexpr bool VEC = FILL == KG_DMA16;
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
    // g * BK * BNP (B). With 16-byte fills, buffer-to-LDS or through
    // registers (U16), each group runs the pipelined main loop (PipeCore)
    // over its slices g, g + KG, g + 2 KG, ...; the ring's barriers are the
    // workgroup's, so every group takes the same number of steps, and a
    // group's slices past the end of K load as zeros. With 4-byte fills
    // (several times as many loads per slice, and more registers in flight)
    // the plain double-buffered loop below is faster: the pipelined one
    // measured 2-5% slower there, and it spilled in the 64x64-wave groups.
    const int nslices = (a.K + BK - 1) / BK;
    if constexpr (FILL == KG_DMA16 || FILL == KG_U16) {
        using Core = PipeCore<BM, BN, WM, WN, BK, 2, VEC, false, TA, TB, FILL == KG_U16>;
        static_assert(Core::NT == GT && Core::LDS_A == BM * BK && Core::LDS_B == BK * BNP,
                      "the group's pipeline works in the group's part of each stage");
        const Core core(a, tm, tn, tl);
        float* const Ast[4] = {As0 + g * BM * BK, As1 + g * BM * BK, nullptr, nullptr};
        float* const Bst[4] = {Bs0 + g * BK * BNP, Bs1 + g * BK * BNP, nullptr, nullptr};
        // Group g has (nslices - g + KG - 1) / KG slices, one fewer than the
        // first groups' when KG does not divide nslices; its last step then
        // multiplies nothing. (The 64x64-wave groups, with 64 accumulators
        // per lane, have no registers to spare for the split-off last step
        // and multiply the zeros.)
        constexpr bool GUARD = PER_LANE <= 32;
        core.template mainloop<KG, GUARD>(a, 0, (nslices + KG - 1) / KG, Ast, Bst, acc, g,
                                          (nslices - g + KG - 1) / KG);
    } else {
        const SubstepMma<BM, BNP, WM, WN, BK, TA, TB> mma(wm, wn, h, c, g * BM * BK, g * BK * BNP);
        auto compute = [&](const float* Ac, const float* Bc) { mma(Ac, Bc, acc); };

        // Step i: group g multiplies slice i*KG + g from the current stage while
        // its loads of slice (i+1)*KG + g fill the other one; one workgroup
        // barrier per step (it also waits for each wave's loads).
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
    }

    // Fixed-order reduction of the four partial tiles (the main loop's last
    // barrier has retired every read of the stages and every load into them).
    // Two-level tree in a fixed order, (p0 + p2) + (p1 + p3), through the
    // stages: each wave holds at most one partial tile besides its own. The
    // accumulators of a lane travel as 16-byte vectors; vector q of thread tl
    // goes to lo[(q*GT + tl)*4] for q < Q/2 and to hi[((q - Q/2)*GT + tl)*4]
    // above, so a wave's accesses are consecutive. Slot 0 is stage 0 and slot
    // 1 stage 1: each half of a slot is its B part when a whole partial tile
    // fits in it, else the A part and the B part.
    // Where they fit in the stages (every tile but the 64x64-wave one), the
    // four groups split the tile by row quarters instead: quarter q is the
    // accumulators 4q .. 4q+3 of every 32x32 block (rows 8q .. 8q+7 of the
    // block), and group q owns it. Each group writes its partial sums of the
    // three quarters it does not own, one barrier, and each group adds the
    // other three groups' partials of its quarter in the same fixed order,
    // (p0 + p2) + (p1 + p3), and stores it: one barrier instead of three,
    // and all waves store. Region (q, s) holds source group s's partials of
    // quarter q (s < q: region 3q + s, else 3q + s - 1), 16 bytes per thread
    // of a group, block by block: a wave's accesses are consecutive.
    constexpr int QQ = BI * BJ;                                 // blocks per lane
    constexpr int RS = QQ * GT * 4;                             // floats per region
    constexpr int NA = (KG * BM * BK) / RS, NB = (KG * BK * BNP) / RS;
    if constexpr (2 * (NA + NB) >= 12) {
        auto region = [&](int r) -> float* {
            return r < NA ? As0 + r * RS
                 : r < NA + NB ? Bs0 + (r - NA) * RS
                 : r < 2 * NA + NB ? As1 + (r - NA - NB) * RS
                 : Bs1 + (r - 2 * NA - NB) * RS;
        };
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bj = 0; bj < BJ; ++bj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (q == g) continue;
                    float* dst = region(3 * q + (g < q ? g : g - 1)) + ((bi * BJ + bj) * GT + tl) * 4;
                    *(f32x4*)dst = f32x4{acc[bi][bj][4 * q], acc[bi][bj][4 * q + 1],
                                         acc[bi][bj][4 * q + 2], acc[bi][bj][4 * q + 3]};
                }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q != g) continue;
#pragma unroll
            for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                for (int bj = 0; bj < BJ; ++bj) {
                    f32x4 p[KG];
#pragma unroll
                    for (int src = 0; src < KG; ++src)
                        p[src] = src == q ? f32x4{acc[bi][bj][4 * q], acc[bi][bj][4 * q + 1],
                                                  acc[bi][bj][4 * q + 2], acc[bi][bj][4 * q + 3]}
                                          : *(const f32x4*)(region(3 * q + (src < q ? src : src - 1)) +
                                                            ((bi * BJ + bj) * GT + tl) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = (p[0][e] + p[2][e]) + (p[1][e] + p[3][e]);
                        const int i = wm * WM + bi * 32 + 8 * q + 4 * h + e;
                        const int j = wn * WN + bj * 32 + c;
                        if (i < rows_valid && j < cols_valid)
                            store_out(a, (int64_t)m0 + i, (int64_t)n0 + j, v);
                    }
                }
        }
        return;
    }
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

// U16: whether calls with rows that are not whole 16-byte chunks take the
// register-staged 16-byte fill (its 16 staging registers must fit the
// occupancy target) rather than 4-byte buffer-to-LDS loads.
#ifndef SGEMM_KG_U16
#define SGEMM_KG_U16 1
#endif
template <int BM, int BN, int WM, int WN, int BK = 16, bool U16 = SGEMM_KG_U16 != 0>
struct KgroupInstance {
    static constexpr int NT = 4 * (BM / WM) * (BN / WN) * 64;
    static constexpr int kBM = BM, kBN = BN, kBK = BK;
    static int check(const Args& a) {
        if (!extents_ok(a, BM, BN, BK)) return SGEMM_F32_ERR_TOO_LARGE;
        const int64_t tiles = cdiv(a.M, BM) * cdiv(a.N, BN);
        return tiles <= max_workgroups(NT) ? 0 : SGEMM_F32_ERR_TOO_LARGE;
    }
    // The fill a call takes: 16-byte buffer-to-LDS loads when every row is
    // whole 16-byte chunks, else 16-byte loads through registers when the
    // extents allow them (U16), else 4-byte buffer-to-LDS loads.
    static int fill(const Args& a) {
        if (vec_ok(a)) return KG_DMA16;
        return (U16 && fillu_ok(a, BM, BN, BK)) ? KG_U16 : KG_DMA4;
    }
    static hipError_t launch(const Args& a, hipStream_t s) {
        const int tm = (int)cdiv(a.M, BM), tn = (int)cdiv(a.N, BN);
        const dim3 grid((unsigned)((int64_t)tm * tn)), block(NT);
        const int f = fill(a);
        return with_trans(a, [&](auto ta, auto tb) {
            constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
            if (f == KG_DMA16)
                hipLaunchKernelGGL((k_mfma_kgroup<BM, BN, WM, WN, BK, KG_DMA16, TA, TB>), grid, block,
                                   0, s, a, tm, tn, xcd_remap_enabled());
            else if (f == KG_U16)
                hipLaunchKernelGGL((k_mfma_kgroup<BM, BN, WM, WN, BK, U16 ? KG_U16 : KG_DMA4, TA, TB>),
                                   grid, block, 0, s, a, tm, tn, xcd_remap_enabled());
            else
                hipLaunchKernelGGL((k_mfma_kgroup<BM, BN, WM, WN, BK, KG_DMA4, TA, TB>), grid, block,
                                   0, s, a, tm, tn, xcd_remap_enabled());
            return hipGetLastError();
        });
    }
    static const void* kernel() { return (const void*)k_mfma_kgroup<BM, BN, WM, WN, BK, KG_DMA16>; }
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
// 96x64 tile, 4 groups of 3 waves of 32x64 (12 waves, 80 KB LDS): the
// 64x96 tile stood on end, for outputs with the odd shape's sides swapped
// (1531x1000 is exactly 256 such tiles).
#ifndef SGEMM_KG96x64_WM
#define SGEMM_KG96x64_WM 32
#define SGEMM_KG96x64_WN 64
#endif
using Kg96x64 = KgroupInstance<96, 64, SGEMM_KG96x64_WM, SGEMM_KG96x64_WN>;
Variant kMfmaKgroup96x64 = {"mfma_96x64_kg4", Kg96x64::check, Kg96x64::launch, Kg96x64::kernel(),
                            Kg96x64::NT, true, nullptr, nullptr, Kg96x64::kBM, Kg96x64::kBN,
                            Kg96x64::kBK};
// 128x128 tile, 4 groups of 4 waves of 64x64 (16 waves, 128 KB LDS): one
// tile per compute unit with four waves per SIMD, for shapes with at most
// about one 128x128 tile per compute unit and long K.
// Its 64x64 waves leave no room for the register stage at four waves per
// SIMD (it spills), so unaligned rows take the 4-byte fill.
using Kg128x128 = KgroupInstance<128, 128, 64, 64, 16, false>;
// Its 16-byte-fill instances with B transposed spill (the automatic choice
// leaves them out).
static bool auto_kg128(const Args& a) { return !(vec_ok(a) && a.tb); }
Variant kMfmaKgroup128 = {"mfma_128x128_kg4", Kg128x128::check, Kg128x128::launch,
                          Kg128x128::kernel(), Kg128x128::NT, true, nullptr, nullptr,
                          Kg128x128::kBM, Kg128x128::kBN, Kg128x128::kBK, auto_kg128};

}  // namespace sgemm
