// Internal interface between the C-ABI layer (api.cpp) and the kernel
// translation units. Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace sgemm {

// Shape/alignment checks a variant runs on the host before launching.
// Return 0, or SGEMM_F32_ERR_UNSUPPORTED / SGEMM_F32_ERR_TOO_LARGE.
typedef int (*check_fn)(const Args&);
typedef hipError_t (*launch_fn)(const Args&, hipStream_t);
// Stream-K variants: workspace bytes a launch needs on a device with `cus`
// compute units, and the launch with that workspace.
typedef size_t (*ws_size_fn)(const Args&, int cus);
typedef hipError_t (*launch_ws_fn)(const Args&, void* ws, size_t ws_bytes, int cus, hipStream_t);

struct Variant {
    const char* name;
    check_fn check;
    launch_fn launch;
    const void* kernel;  // main kernel, for hipFuncGetAttributes / occupancy
    int threads;         // workgroup size of the main kernel
    bool trans_ok;       // accepts transposed operands (Args::ta, Args::tb)
    // Stream-K variants only (else null): `launch` is then unused.
    ws_size_fn ws_size;
    launch_ws_fn launch_ws;
    // Matrix-core tile kernels the dispatch model chooses among: the output
    // tile of one workgroup and the K slice of one pipeline step (the unit
    // of a stream-K split). 0 for the other variants.
    int bm = 0, bn = 0, bk = 0;
    // Whether the automatic choice may launch this variant for the call:
    // false when the kernel instance the call would take (its fill, whole
    // tiles or not, transpositions) spills registers to scratch memory, as
    // the compiler's resource remarks show. Null: every instance qualifies.
    // A CPU test checks every spilling instance of the build against these.
    bool (*auto_ok)(const Args&) = nullptr;
};

// ---------------------------------------------------------------------------
// Host side of the stream-K split (SkPlan in common.hpp). With T tiles of
// S slices on C compute units, floor(T / C) * C tiles stay whole, so that
// every unit gets the same number of whole tiles; the R = T mod C remaining
// tiles are split. Their R*S slices go to G = min(C, 4R) workgroups in runs
// of ceil(R*S / G) slices, which keeps a tile to about four pieces, as the
// pages found best ("Optimizing Matrix Multiply on CUDA, Part 2",
// "Distributing the Partially Filled Wave": two to four pieces; sixteen
// lost). Workgroups left without slices by the rounding are not launched.
// R == 0, or more slices than 32-bit indexing allows, gives no split.
// Since G >= R, a run holds at most `slices` slices (upw <= slices), so it
// touches at most two tiles, which the kernel relies on.
// ---------------------------------------------------------------------------
struct SkSplit {
    int64_t tiles = 0, slices = 0;
    int64_t dp_tiles = 0, sk_tiles = 0, sk_wgs = 0, upw = 0;
    bool split() const { return sk_tiles > 0; }
    // Tiles' worth of work on the busiest compute unit.
    double busiest_tiles(int cus) const {
        if (!split()) return (double)((tiles + cus - 1) / (cus > 0 ? cus : 1));
        return (double)(dp_tiles / cus) + (double)upw / (double)slices;
    }
};

inline SkSplit sk_split(int64_t tiles, int64_t slices, int cus) {
    SkSplit p;
    p.tiles = tiles;
    p.slices = slices;
    if (cus < 1) cus = 1;
    const int64_t R = tiles % cus;
    p.dp_tiles = tiles - R;
    if (R == 0 || slices < 1 || R * slices > INT32_MAX) {
        p.dp_tiles = tiles;
        return p;
    }
    const int64_t G = R * 4 < cus ? R * 4 : cus;
    const int64_t U = R * slices;
    p.upw = (U + G - 1) / G;
    p.sk_wgs = (U + p.upw - 1) / p.upw;
    p.sk_tiles = R;
    return p;
}

// Workspace: the partial tiles, two slots per stream-K workgroup.
inline size_t sk_workspace_bytes(const SkSplit& p, int bm, int bn) {
    if (!p.split()) return 0;
    return (size_t)(2 * p.sk_wgs) * (size_t)bm * (size_t)bn * sizeof(float);
}


// C = beta*C (K == 0 or alpha == 0), C read only when beta != 0.
hipError_t launch_scale(const Args& a, hipStream_t s);

// Variant descriptors (not const: clang would otherwise treat these
// constant-initialised globals as usable from device code and try to resolve
// their host function pointers in the device link). Read-only after load.
// ladder.hip
extern Variant kNaive, kCoalesced, kLdsTiled, kReg1d, kReg2d, kVec4TransA;
// valu_main.hip
extern Variant kValuMain;
// mfma_pipe.hip, mfma_kgroup.hip, mfma_small.hip
extern Variant kMfma128, kMfma64, kMfmaSkinny, kMfmaKsplit, kMfmaDirect, kMfma64x128,
    kMfma256, kMfmaKgroup, kMfmaKgroup96, kMfmaKgroup96x64, kMfmaKgroup128, kMfma128Sk, kMfma64x128Sk, kMfma256Sk;

// Common host checks.
bool aligned16(const void* p);
// Whether the tiled matrix-core kernels can fill both operands with 16-byte
// loads: the contiguous extent of each operand (K of A, N of B; M of a
// transposed A, K of a transposed B), both leading dimensions and both base
// addresses in whole 16-byte chunks. Otherwise they use 4-byte loads, and the
// dispatch model applies each kernel's 4-byte-fill factor.
bool vec_ok(const Args& a);
// Largest workgroup count a 1-D dispatch of `threads`-lane workgroups allows.
int64_t max_workgroups(int threads);
// 1 unless the environment sets SGEMM_F32_XCD_REMAP=0 (for measuring the
// XCD-aware tile order against plain dispatch order).
int xcd_remap_enabled();

}  // namespace sgemm
