// The pipelined FP32 matrix-core kernel (k_mfma_pipe, body PipeCore) and its
// instances: mfma_256x256, mfma_128x128, mfma_64x128 and mfma_64x64, with the
// stream-K forms of the first three (k_mfma_pipe_sk, summed by k_sk_fixup). Operand layouts and edge
// handling: mfma_common.hpp.
#include "mfma_pipecore.hpp"

namespace sgemm {

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
constexpr int M128_WM = SGEMM_M128_WM, M128_WN = SGEMM_M128_WN;

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

template <int BM, int BN, int WM, int WN, int BK, int STAGES, int WPE, bool VEC, bool FULL,
          bool TA = false, bool TB = false, bool U16 = false>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void k_mfma_pipe(Args a, int tiles_m, int tiles_n, int xcd_remap) {
    using Core = PipeCore<BM, BN, WM, WN, BK, STAGES, VEC, FULL, TA, TB, U16>;
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
          bool TA = false, bool TB = false, bool U16 = false>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void k_mfma_pipe_sk(Args a, int tiles_m, int tiles_n, int xcd_remap, SkPlan p) {
    using Core = PipeCore<BM, BN, WM, WN, BK, STAGES, VEC, FULL, TA, TB, U16>;
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
    const int u0 = j * p.upw;
    const int u_end = (u0 + p.upw) < U ? (u0 + p.upw) : U;
    // A run holds at most one tile's worth of slices (upw <= slices, see
    // sk_split), so it touches at most two tiles: the rest of the tile it
    // starts in, then the start of the next. Each piece is a straight-line
    // block of its own (as a loop, the compiler kept per-lane values of one
    // iteration live into the next and spilled them).
    auto piece = [&](int u, int tid) {
        const int st = u / p.slices;
        const int s0 = u - st * p.slices;
        const int s1 = (s0 + (u_end - u)) < p.slices ? (s0 + (u_end - u)) : p.slices;
        tile_of_first(p.dp_tiles + st, p.dp_tiles, tiles_m, tiles_n, M128_GROUP_M,
                      xcd_remap != 0, tm, tn);
        const Core core(a, tm, tn, tid);
        Core::zero(acc);
        core.mainloop(a, s0, s1, Ast, Bst, acc);
        if (s0 == 0 && s1 == p.slices)
            core.store(a, acc);
        else
            Io::put(p.partials + (size_t)sk_slot(p, j, st) * BM * BN, core.t, acc);
        return u + (s1 - s0);
    };
    if (u0 >= u_end) return;
    const int u1 = piece(u0, threadIdx.x);
    if (u1 >= u_end) return;
    // The second piece's per-lane offsets derive from the thread index;
    // hidden from the compiler here, they are recomputed rather than kept
    // live (and spilled) across the first piece.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    piece(u1, tid);
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

bool vec_ok(const Args& a) {
    const int ca = a.ta ? a.M : a.K, cb = a.tb ? a.K : a.N;
    return !((ca & 3) || (cb & 3) || (a.lda & 3) || (a.ldb & 3) || !aligned16(a.A) ||
             !aligned16(a.B));
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
// cover the problem: no range masks) or the masked one, and the fill: 16-byte
// buffer-to-LDS loads when every operand row is whole 16-byte chunks
// (vec_ok); else, with U16OK and extents that allow it (fillu_ok), 16-byte
// loads through registers; else 4-byte buffer-to-LDS loads. The 4-byte-fill form keeps more loads in flight per
// lane; it targets 3 waves per SIMD (at 4 it would spill), or as many as one
// workgroup puts on each SIMD if that is more: the 256x256 tile's 16 waves
// need 4, so its 4-byte forms spill and the automatic choice leaves them out
// (auto_vec below); it has no registers to spare for U16 either. U16_TB:
// U16 also when B is stored transposed (the 128x128 tile spills there).
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int WPE, bool U16OK = false,
          bool U16_TB = true>
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
    // f(VEC, FULL, TA, TB, U16), each a std::integral_constant<bool>; U16 only
    // with `u16`.
    template <class F>
    static hipError_t forms(const Args& a, bool u16, F&& f) {
        using T = std::true_type;
        using N = std::false_type;
        const bool vec = vec_ok(a);
        const bool full = a.M % BM == 0 && a.N % BN == 0 && a.K % BK == 0;
        const bool reg = U16OK && u16 && !vec && fillu_ok(a, BM, BN, BK);
        return with_trans(a, [&](auto ta, auto tb) {
            if (vec && full) return f(T{}, T{}, ta, tb, N{});
            if (vec) return f(T{}, N{}, ta, tb, N{});
            if constexpr (U16OK && (U16_TB || !decltype(tb)::value))
                if (reg) return f(N{}, N{}, ta, tb, T{});
            return f(N{}, N{}, ta, tb, N{});
        });
    }
    static hipError_t launch(const Args& a, hipStream_t s) {
        const int tm = (int)cdiv(a.M, BM), tn = (int)cdiv(a.N, BN);
        const dim3 grid((unsigned)((int64_t)tm * tn)), block(NT);
        return forms(a, true, [&](auto vec, auto full, auto ta, auto tb, auto u16) {
            constexpr bool V = decltype(vec)::value, F = decltype(full)::value;
            constexpr bool U = decltype(u16)::value;
            hipLaunchKernelGGL((k_mfma_pipe<BM, BN, WM, WN, BK, STAGES, (V || U) ? WPE : WPE4, V, F,
                                            decltype(ta)::value, decltype(tb)::value, U>),
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
        const hipError_t e = forms(a, true, [&](auto vec, auto full, auto ta, auto tb, auto u16) {
            constexpr bool V = decltype(vec)::value, F = decltype(full)::value;
            constexpr bool U = decltype(u16)::value;
            hipLaunchKernelGGL((k_mfma_pipe_sk<BM, BN, WM, WN, BK, STAGES, (V || U) ? WPE : WPE4, V,
                                               F, decltype(ta)::value, decltype(tb)::value, U>),
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

// mfma_64x64 tile parameters: a 64x64 block tile of 4 waves of 32x32 (one
// 32x32 MFMA block each), 32-deep K slices, two 16 KiB LDS stages, so five
// workgroups share a compute unit: four times the tiles of mfma_128x128 for
// shapes whose 128x128 grid leaves compute units idle.
#ifndef SGEMM_M64_BK
#define SGEMM_M64_BK 32
#endif
#ifndef SGEMM_M64_WPE
#define SGEMM_M64_WPE 5
#endif

using Pipe256 = PipeInstance<SGEMM_M256_BM, SGEMM_M256_BN, SGEMM_M256_WM, SGEMM_M256_WN,
                             SGEMM_M256_BK, SGEMM_M256_STAGES, SGEMM_M256_WPE>;
using Pipe128 = PipeInstance<M128_BM, M128_BN, M128_WM, M128_WN, M128_BK, 2,
                             SGEMM_M128_WAVES_PER_EU, true, false>;
// Two 24 KiB LDS stages per 4-wave workgroup: three workgroups per compute
// unit, so three waves per SIMD.
using Pipe64x128 =
    PipeInstance<64, 128, SGEMM_M64x128_WM, SGEMM_M64x128_WN, SGEMM_M64x128_BK, 2, 3, true>;
using Pipe64 = PipeInstance<64, 64, 32, 32, SGEMM_M64_BK, 2, SGEMM_M64_WPE, true>;

// Instances the automatic choice may launch: the spill-free ones. At four
// waves per SIMD (128 registers) the 256x256 tile's 4-byte fills spill, and
// so do its stream-K form's 4-byte fills and masked 16-byte fills (except
// with only B transposed); the 64x128 stream-K kernel's 4-byte fills (taken
// only when the register-staged fill cannot run) spill when A is read
// untransposed.
static bool auto_vec(const Args& a) { return vec_ok(a); }
static bool auto_256_sk(const Args& a) {
    const bool full = a.M % 256 == 0 && a.N % 256 == 0 && a.K % SGEMM_M256_BK == 0;
    return vec_ok(a) && (full || (a.tb && !a.ta));
}
static bool auto_64x128_sk(const Args& a) { return vec_ok(a) || fillu_ok(a, 64, 128, 32) || a.ta; }

Variant kMfma256 = {"mfma_256x256", Pipe256::check, Pipe256::launch, Pipe256::kernel(),
                    Pipe256::NT, true, nullptr, nullptr, Pipe256::kBM, Pipe256::kBN, Pipe256::kBK,
                    auto_vec};
Variant kMfma128 = {"mfma_128x128", Pipe128::check, Pipe128::launch, Pipe128::kernel(),
                    Pipe128::NT, true, nullptr, nullptr, Pipe128::kBM, Pipe128::kBN, Pipe128::kBK};
// 64x128: twice the tiles of mfma_128x128 for medium shapes (e.g. 3072^3,
// whose 576 tiles of 128x128 leave the second round of workgroups a third
// full).
Variant kMfma64x128 = {"mfma_64x128", Pipe64x128::check, Pipe64x128::launch,
                       Pipe64x128::kernel(), Pipe64x128::NT, true, nullptr, nullptr,
                       Pipe64x128::kBM, Pipe64x128::kBN, Pipe64x128::kBK};
Variant kMfma64 = {"mfma_64x64", Pipe64::check, Pipe64::launch, Pipe64::kernel(), Pipe64::NT,
                   true, nullptr, nullptr, Pipe64::kBM, Pipe64::kBN, Pipe64::kBK};
// Stream-K forms (they need a workspace: sgemm_f32_ws).
Variant kMfma256Sk = {"mfma_256x256_sk", Pipe256::check, nullptr, Pipe256::sk_kernel(),
                      Pipe256::NT, true, Pipe256::ws_size, Pipe256::launch_ws,
                      Pipe256::kBM, Pipe256::kBN, Pipe256::kBK, auto_256_sk};
Variant kMfma128Sk = {"mfma_128x128_sk", Pipe128::check, nullptr, Pipe128::sk_kernel(),
                      Pipe128::NT, true, Pipe128::ws_size, Pipe128::launch_ws,
                      Pipe128::kBM, Pipe128::kBN, Pipe128::kBK};
Variant kMfma64x128Sk = {"mfma_64x128_sk", Pipe64x128::check, nullptr, Pipe64x128::sk_kernel(),
                         Pipe64x128::NT, true, Pipe64x128::ws_size, Pipe64x128::launch_ws,
                         Pipe64x128::kBM, Pipe64x128::kBN, Pipe64x128::kBK, auto_64x128_sk};

}  // namespace sgemm
