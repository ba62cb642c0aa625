// Shared pieces of the gfx950 SGEMM kernels: the argument block, the
// epilogue, buffer-resource loads with out-of-range-reads-zero, and the
// workgroup -> output-tile mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm {

// One GEMM problem, passed by value as the kernel argument block.
// Row-major: A(i,k) = A[i*lda + k], B(k,j) = B[k*ldb + j], C(i,j) = C[i*ldc + j]
// (untransposed operands).
struct Args {
    const float* A;
    const float* B;
    float* C;
    int64_t lda, ldb, ldc;
    int32_t M, N, K;
    float alpha, beta;
    // Transposed operands (only kernels whose variant sets trans_ok read
    // these): ta -> A is stored K x M, A(i,k) = A[k*lda + i]; tb -> B is
    // stored N x K, B(k,j) = B[j*ldb + k].
    int32_t ta, tb;
    // C stored column-major, C(i,j) = C[j*ldc + i] (only mfma_skinny, which
    // takes column-major calls with few rows unswapped, writes it this way).
    int32_t tc;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Epilogue for one output: C = alpha*acc + beta*C0, where C0 is read only
// when beta != 0 (so an uninitialised C cannot leak NaN into the result).
__device__ __forceinline__ void store_out(const Args& a, int64_t i, int64_t j, float acc) {
    float* p = a.C + i * a.ldc + j;
    float v = a.alpha * acc;
    if (a.beta != 0.0f) v = __builtin_fmaf(a.beta, *p, v);
    *p = v;
}
// The same for a column-major C (Args::tc).
__device__ __forceinline__ void store_out_col(const Args& a, int64_t i, int64_t j, float acc) {
    float* p = a.C + j * a.ldc + i;
    float v = a.alpha * acc;
    if (a.beta != 0.0f) v = __builtin_fmaf(a.beta, *p, v);
    *p = v;
}

// ---------------------------------------------------------------------------
// Buffer resources. A raw buffer load whose byte offset is at or past the
// resource's num_records returns zeros instead of touching memory, which is
// how the tiled kernels fill the parts of a tile that hang off the matrix:
// every masked element gets the offset OOB, far past any extent the host
// allows (extents are checked to stay below 2^31 bytes).
// ---------------------------------------------------------------------------
constexpr uint32_t OOB = 0x80000000u;
// Third descriptor word for gfx9-family raw buffers: 32-bit data format,
// no swizzle, no index stride.
constexpr int RSRC_FLAGS = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes,
                                             RSRC_FLAGS);
}

__device__ __forceinline__ f32x4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ float buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// Buffer load straight into LDS (no VGPR round trip): every lane's 16 (or 4)
// bytes land at lds_base + 16 (or 4) * lane, lds_base being wave-uniform. Out-of-
// range offsets write zeros, as for the register loads.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, const float* lds_base,
                                               uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds_base), 16, (int)off, 0, 0, 0);
}

__device__ __forceinline__ void buf_load_lds4(__amdgpu_buffer_rsrc_t r, const float* lds_base,
                                              uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds_base), 4, (int)off, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Workgroup id -> (tile row, tile column).
//
// MI355X spreads consecutive workgroup ids of a dispatch round-robin over its
// 8 XCDs, each with its own L2. The mapping first renumbers ids so that each
// XCD receives one contiguous range of logical ids, then walks the tile grid
// in column-major order within bands of `group_m` tile rows, so that the
// workgroups that run together on one XCD cover a compact block of C and
// share their A row panels and B column panels in that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int NUM_XCD = 8;

// tile_of_first: the renumbering applies to the ids below `first` only (a
// bijection of [0, first)); ids from `first` on keep their order. The
// stream-K kernels use it for their whole-tile workgroups.
__device__ __forceinline__ void tile_of_first(int wg, int first, int tiles_m, int tiles_n,
                                              int group_m, bool xcd_remap, int& tm, int& tn) {
    int L = wg;
    if (xcd_remap && wg < first) {
        const int x = wg % NUM_XCD, idx = wg / NUM_XCD;
        const int q = first / NUM_XCD, r = first % NUM_XCD;
        L = x * q + (x < r ? x : r) + idx;
    }
    const int per_group = group_m * tiles_n;
    const int g = L / per_group;
    const int first_m = g * group_m;
    const int rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in = L - g * per_group;
    tm = first_m + in % rows;
    tn = in / rows;
}

__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int group_m,
                                        bool xcd_remap, int& tm, int& tn) {
    tile_of_first(wg, tiles_m * tiles_n, tiles_m, tiles_n, group_m, xcd_remap, tm, tn);
}

// ---------------------------------------------------------------------------
// Stream-K work split (kernel argument of the stream-K kernels). Following
// the pages' hybrid ("Optimizing Matrix Multiply on CUDA, Part 2",
// "Distributing the Partially Filled Wave"), the tiles that fill whole rounds
// of the compute units stay whole, and only the remaining tiles are split
// along K: their slices, taken tile by tile, are dealt out in equal
// contiguous runs to sk_wgs workgroups; the pieces of each split tile are
// then summed in K order and written to C.
//   workgroups [0, dp_tiles)                whole tiles 0 .. dp_tiles-1
//   workgroups dp_tiles + j, j < sk_wgs     slices [j*upw, min((j+1)*upw, U))
//                                           of tiles dp_tiles .. dp_tiles+sk_tiles-1,
//                                           U = sk_tiles * slices, slice u in
//                                           tile dp_tiles + u / slices
// A workgroup's run crosses a tile boundary at most at its two ends, so it
// has at most two partial pieces: its first (slot 2j) and its last (slot
// 2j+1), each a BM x BN tile of partial sums in `partials`.
// ---------------------------------------------------------------------------
struct SkPlan {
    int dp_tiles, sk_tiles, sk_wgs, upw, slices;
    float* partials;   // 2 * sk_wgs slots of BM*BN floats
};

// LDS swizzle for a 16-float row of an untransposed A tile read with 16-byte
// loads: 16-byte chunk q of row r is stored at chunk q ^ swz16(r). With 8
// consecutive lanes on 8 consecutive rows (fragment reads) or 4 lanes per row
// on 2-4 consecutive rows (tile fills), every 16-byte access of a lane group
// lands in a distinct bank group for both a 32-bank and a 64-bank LDS.
__device__ __forceinline__ int swz16(int r) { return ((r >> 2) ^ (r & 2)) & 3; }

// The same for 32-float rows (8 chunks): 8 consecutive rows, or the even and
// the odd rows of 16 consecutive rows, map a fixed logical chunk to distinct
// physical chunks, and 8 lanes filling one row hit 8 distinct chunks.
__device__ __forceinline__ int swz32(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// For 64-float rows (16 chunks) the row index itself spreads any 8 or 16
// consecutive rows over distinct chunks.
__device__ __forceinline__ int swz64(int r) { return r & 15; }

template <int BK>
__device__ __forceinline__ int swz_chunk(int r) {
    static_assert(BK == 16 || BK == 32 || BK == 64, "A tile rows are 16, 32 or 64 floats");
    return BK == 16 ? swz16(r) : (BK == 32 ? swz32(r) : swz64(r));
}

}  // namespace sgemm
