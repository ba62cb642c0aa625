// Internal interface between the C-ABI layer (api.cpp) and the kernel
// translation units. Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace sgemm {

// Shape/alignment checks a variant runs on the host before launching.
// Return 0, or SGEMM_F32_ERR_UNSUPPORTED / SGEMM_F32_ERR_TOO_LARGE.
typedef int (*check_fn)(const Args&);
typedef hipError_t (*launch_fn)(const Args&, hipStream_t);

struct Variant {
    const char* name;
    check_fn check;
    launch_fn launch;
    const void* kernel;  // main kernel, for hipFuncGetAttributes / occupancy
    int threads;         // workgroup size of the main kernel
    bool trans_ok;       // accepts transposed operands (Args::ta, Args::tb)
};

// C = beta*C (K == 0 or alpha == 0), C read only when beta != 0.
hipError_t launch_scale(const Args& a, hipStream_t s);

// Variant descriptors (not const: clang would otherwise treat these
// constant-initialised globals as usable from device code and try to resolve
// their host function pointers in the device link). Read-only after load.
// ladder.hip
extern Variant kNaive, kCoalesced, kLdsTiled, kReg1d, kReg2d, kVec4TransA;
// valu_main.hip
extern Variant kValuMain;
// mfma.hip
extern Variant kMfma128, kMfma64, kMfmaSkinny, kMfmaKsplit, kMfmaDirect, kMfma64x128,
    kMfma256, kMfmaKgroup, kMfmaKgroup96, kMfmaKgroup128;

// Common host checks.
bool aligned16(const void* p);
// Largest workgroup count a 1-D dispatch of `threads`-lane workgroups allows.
int64_t max_workgroups(int threads);
// 1 unless the environment sets SGEMM_F32_XCD_REMAP=0 (for measuring the
// XCD-aware tile order against plain dispatch order).
int xcd_remap_enabled();

}  // namespace sgemm
