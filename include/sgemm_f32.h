/*
 * sgemm_f32 -- single-precision general matrix multiply for AMD MI355X (gfx950).
 *
 *   C = alpha * A * B + beta * C          (row-major, FP32 in, FP32 accumulate, FP32 out)
 *
 * The operation is the one every source page builds toward: each output
 * C[i][j] is alpha times the K-term dot product of row i of A and column j of
 * B, plus beta times the old C[i][j] ("GEMM from scratch", Module 02, "One
 * Thread Per Output"; "Optimizing Matrix Multiply on CUDA, Part 1", "Counting
 * the Work"). The arithmetic is plain FP32 -- no TF32-style or reduced
 * precision inputs ("100 Days of GPU, Day 44", "The honest target": FP32 in,
 * FP32 compute type, FP32 out). The status-code return mirrors the library
 * call those pages score against (Day 44, "Five paths, one table").
 *
 * Layout (all three matrices row-major, element (r, c) at base[r * ld + c]):
 *   A : M x K, leading dimension lda >= max(1, K)
 *   B : K x N, leading dimension ldb >= max(1, N)
 *   C : M x N, leading dimension ldc >= max(1, N)
 * A, B and C are device pointers owned by the caller; they must be 4-byte
 * aligned. C must not overlap A or B. The library allocates no memory on the
 * call path and keeps no per-call state.
 *
 * Semantics the pages leave open (BLAS conventions):
 *   - M == 0 or N == 0: returns 0 and touches no memory.
 *   - K == 0 or alpha == 0: A and B are not read; C = beta * C.
 *   - beta == 0: C is write-only (its old contents, even NaN, are ignored).
 *   - Summation order is unspecified; results are deterministic for a given
 *     device, variant and input (no atomics). FP32 fused multiply-adds are used.
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without synchronizing.
 *
 * Return codes (int):
 *     0                     success
 *    -i  (i = 1..11)        argument i of sgemm_f32 is invalid, counting M as 1:
 *                           1 M<0, 2 N<0, 3 K<0, 5 A null or misaligned,
 *                           6 lda too small, 7 B null or misaligned, 8 ldb too
 *                           small, 10 C null or misaligned, 11 ldc too small.
 *                           (A, B, C are only required when they are read or
 *                           written.) sgemm_f32_variant uses the same numbers,
 *                           and so do the _ex entry points for these arguments
 *                           (named by meaning, not position), plus
 *                           -13 layout, -14 transa, -15 transb.
 *    SGEMM_F32_ERR_VARIANT      variant id out of range
 *    SGEMM_F32_ERR_UNSUPPORTED  the forced variant cannot run this shape or
 *                               alignment (e.g. a 16-byte-load rung with a
 *                               leading dimension that is not a multiple of 4)
 *    SGEMM_F32_ERR_TOO_LARGE    a size exceeds what the kernel can index
 *    SGEMM_F32_ERR_DEVICE       no usable HIP device
 *    SGEMM_F32_ERR_WORKSPACE    a forced stream-K variant was given less
 *                               workspace than sgemm_f32_ws_size reports
 *    -16                    (the _ws entry points) the workspace pointer is
 *                           NULL with a nonzero size, or not 16-byte aligned
 *    SGEMM_F32_ERR_SCRATCH  (sgemm_f32_ws_static) the forced stream-K variant
 *                           needs more than the fixed scratch holds
 *   > 0                     a hipError_t reported by the HIP runtime at launch
 *
 * Thread safety: all entry points are reentrant, except that calls of
 * sgemm_f32_ws_static whose executions overlap on one GPU share its scratch
 * (see there).
 */
#ifndef SGEMM_F32_H
#define SGEMM_F32_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SGEMM_F32_API __attribute__((visibility("default")))
#else
#define SGEMM_F32_API
#endif

#define SGEMM_F32_OK 0
#define SGEMM_F32_ERR_VARIANT (-100)
#define SGEMM_F32_ERR_UNSUPPORTED (-101)
#define SGEMM_F32_ERR_TOO_LARGE (-102)
#define SGEMM_F32_ERR_DEVICE (-103)
#define SGEMM_F32_ERR_WORKSPACE (-104)
#define SGEMM_F32_ERR_SCRATCH (-105)

/* Size of the fixed device scratch behind sgemm_f32_ws_static (32 MiB). */
#define SGEMM_F32_SCRATCH_BYTES (32u * 1024u * 1024u)

/* Kernel variants. The first six are the rungs of the pages' optimisation
 * ladder, rebuilt for wave64; the rest are the gfx950 kernels the automatic
 * dispatch chooses from. Every variant computes the same product. */
enum sgemm_f32_variant_id {
    /* one lane per output, consecutive lanes walk down a column of C
       ("GEMM from scratch", Module 02) */
    SGEMM_F32_NAIVE = 0,
    /* consecutive lanes take consecutive columns of C (Module 03) */
    SGEMM_F32_COALESCED = 1,
    /* 16x16 tiles of A and B staged in LDS (Module 04; Day 44 step 3) */
    SGEMM_F32_LDS_TILED = 2,
    /* each lane owns a column of 8 outputs (Module 05; Day 44 step 4) */
    SGEMM_F32_REG_1D = 3,
    /* 128x128 block tile, 8x8 outputs per lane (Module 05; Day 44 step 5;
       Part 1, "Stage 3: Register Tiling") */
    SGEMM_F32_REG_2D = 4,
    /* plus 16-byte loads and a transposed A tile, unpadded (Module 06;
       Day 44 step 6); needs 16-byte aligned rows */
    SGEMM_F32_VEC4_TRANSA = 5,
    /* vector-FMA main kernel: wave64 warp tiles, double-buffered K loop,
       conflict-free transposed A tile (Part 2 of "Optimizing Matrix
       Multiply on CUDA") */
    SGEMM_F32_VALU_MAIN = 6,
    /* FP32 matrix-core kernel, 128x128 block tile of 8 waves of 64x32
       (v_mfma_f32_32x32x2_f32), 32-deep K slices in a ring of two LDS
       stages filled by buffer-to-LDS loads, software-pipelined as
       MFMA_256 */
    SGEMM_F32_MFMA_128 = 7,
    /* FP32 matrix-core kernel, 64x64 block tile of 4 waves of 32x32
       (v_mfma_f32_32x32x2_f32), 32-deep K slices, pipelined as MFMA_256,
       five workgroups per compute unit: for shapes with few 128x128 tiles */
    SGEMM_F32_MFMA_64 = 8,
    /* FP32 matrix-core kernel for M <= a few tens of rows (near-GEMV): 16-row
       tiles, the K loop split across the waves of a workgroup */
    SGEMM_F32_MFMA_SKINNY = 9,
    /* FP32 matrix-core kernel, 64x64 tile whose 4 waves split each 64-deep K
       slice four ways and sum their partial tiles in a fixed order (few tiles,
       long K) */
    SGEMM_F32_MFMA_64_K4 = 10,
    /* FP32 matrix-core kernel for small shapes: 32x32 tiles, eight
       waves split K and load their operands straight into matrix-core
       registers (no LDS tile, no barrier in the K loop), fixed-order
       reduction at the end; also a dispatch-model kernel where its grid
       holds one or two tiles per compute unit */
    SGEMM_F32_MFMA_DIRECT = 11,
    /* FP32 matrix-core kernel, 64x128 block tile (4 waves of 64x32,
       v_mfma_f32_32x32x2_f32, 32-deep K slices), pipelined as MFMA_256:
       twice the tiles of mfma_128x128 for medium shapes */
    SGEMM_F32_MFMA_64x128 = 12,
    /* FP32 matrix-core kernel, 256x256 block tile of 16 waves (one
       workgroup per compute unit), software-pipelined: the LDS reads of one
       half slice overlap the MFMAs of the other, and the barrier sits
       between the halves; for large shapes */
    SGEMM_F32_MFMA_256 = 13,
    /* FP32 matrix-core kernel, 64x128 block tile of 16 waves in four K-groups
       (group g takes slices g, g+4, ...), partial tiles summed through LDS in
       a fixed order; for shapes with fewer tiles than compute units */
    SGEMM_F32_MFMA_64x128_KG4 = 14,
    /* the same with a 64x96 tile of 12 waves (4 groups of 3 waves of 64x32) */
    SGEMM_F32_MFMA_64x96_KG4 = 15,
    /* the same with a 128x128 tile of 16 waves (4 groups of 4 waves of 64x64) */
    SGEMM_F32_MFMA_128x128_KG4 = 16,
    /* stream-K forms of MFMA_128 and MFMA_64x128 (sgemm_f32_ws): the tiles
       that fill whole rounds of the compute units are computed whole; the
       rest are split along K across the units, which leave their partial
       tiles in the workspace, and a second kernel sums each tile's pieces
       in K order and writes C. They need a workspace (sgemm_f32_ws_size) */
    SGEMM_F32_MFMA_128_SK = 17,
    SGEMM_F32_MFMA_64x128_SK = 18,
    /* the same for MFMA_256 (one workgroup per compute unit, so whole tiles
       come in rounds of one tile per unit) */
    SGEMM_F32_MFMA_256_SK = 19,
    /* MFMA_64x96_KG4's tile stood on end: 96x64, 12 waves (4 groups of 3
       waves of 32x64); a 1531x1000 output (the column-major 1000x1531 call
       after the swap) is exactly 256 such tiles */
    SGEMM_F32_MFMA_96x64_KG4 = 20,
    SGEMM_F32_NUM_VARIANTS = 21
};

/* Storage order and operand transposition of the _ex entry points (the
 * BLAS sgemm surface). */
enum sgemm_f32_layout {
    SGEMM_F32_ROW_MAJOR = 0, /* element (r, c) at base[r * ld + c] */
    SGEMM_F32_COL_MAJOR = 1  /* element (r, c) at base[c * ld + r] */
};
enum sgemm_f32_trans {
    SGEMM_F32_NO_TRANS = 0, /* op(X) = X */
    SGEMM_F32_TRANS = 1     /* op(X) = X^T */
};

/* C = alpha*A*B + beta*C, kernel chosen automatically (see sgemm_f32_plan). */
SGEMM_F32_API int sgemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                            int64_t lda, const float *B, int64_t ldb, float beta, float *C,
                            int64_t ldc, void *stream);

/* Same operation and return codes, with the kernel forced to `variant`. */
SGEMM_F32_API int sgemm_f32_variant(int variant, int64_t M, int64_t N, int64_t K, float alpha,
                                    const float *A, int64_t lda, const float *B, int64_t ldb,
                                    float beta, float *C, int64_t ldc, void *stream);

/* The variant sgemm_f32 would launch for these arguments on a device with
 * `num_cus` compute units. Host-only: reads no memory through A, B or C (only
 * their addresses, for alignment) and makes no HIP call. Writes the variant
 * id to *variant and returns 0, or returns the same argument errors as
 * sgemm_f32 (-12 if variant is NULL). For a quick-return case (M, N == 0,
 * K == 0 or alpha == 0) *variant is set to -1. */
SGEMM_F32_API int sgemm_f32_plan(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                                 int64_t lda, const float *B, int64_t ldb, float beta,
                                 const float *C, int64_t ldc, int num_cus, int *variant);

/* C = alpha * op(A) * op(B) + beta * C with op(A) M x K, op(B) K x N and C
 * M x N, all three stored in `layout` order (SGEMM_F32_ROW_MAJOR or
 * SGEMM_F32_COL_MAJOR); transa / transb are SGEMM_F32_NO_TRANS or
 * SGEMM_F32_TRANS. The stored matrices are A: M x K (K x M if transa),
 * B: K x N (N x K if transb), C: M x N, and each leading dimension must be at
 * least max(1, the stored matrix's column count) for row-major storage, its
 * row count for column-major storage (CBLAS conventions). Everything else --
 * ownership, alignment, quick returns, beta == 0, asynchrony, return codes --
 * is as for sgemm_f32; sgemm_f32_ex(SGEMM_F32_ROW_MAJOR, SGEMM_F32_NO_TRANS,
 * SGEMM_F32_NO_TRANS, ...) is sgemm_f32.
 *
 * A column-major call is the row-major product of the transposes,
 * C^T = op(B)^T op(A)^T, with the operands and M, N swapped: column-major
 * storage of a matrix is row-major storage of its transpose. This is the
 * operand swap the pages use to get a row-major product out of a
 * column-major library ("100 Days of GPU", Day 44, "Five paths, one table",
 * the library call the page scores against), here applied in the other
 * direction. So a column-major call with both operands
 * untransposed runs the same kernels as a row-major one, at the same speed.
 * After the swap an operand may be stored transposed (A as K x M or B as
 * N x K, row-major); the matrix-core tile kernels read such operands
 * directly (the buffer-to-LDS fill stores them in the LDS layout the
 * fragment reads need; see sgemm_f32_variant_trans_ok), as do mfma_skinny
 * and mfma_direct (whose lanes load their k-runs straight from memory), and
 * the automatic choice then takes one of them. A product with few columns
 * (row-major N <= 32 < M, or column-major M <= 32 < N, which the swap makes
 * one) runs instead as its transpose, which has few rows, on mfma_skinny:
 * A and B are read with their transposition flags flipped and C is written
 * transposed. */
SGEMM_F32_API int sgemm_f32_ex(int layout, int transa, int transb, int64_t M, int64_t N, int64_t K,
                               float alpha, const float *A, int64_t lda, const float *B,
                               int64_t ldb, float beta, float *C, int64_t ldc, void *stream);

/* sgemm_f32_ex with the kernel forced to `variant`. A variant that cannot
 * read a transposed operand (sgemm_f32_variant_trans_ok == 0) returns
 * SGEMM_F32_ERR_UNSUPPORTED when one remains after the column-major swap. */
SGEMM_F32_API int sgemm_f32_variant_ex(int variant, int layout, int transa, int transb, int64_t M,
                                       int64_t N, int64_t K, float alpha, const float *A,
                                       int64_t lda, const float *B, int64_t ldb, float beta,
                                       float *C, int64_t ldc, void *stream);

/* The variant sgemm_f32_ex would launch, as sgemm_f32_plan (host-only). */
SGEMM_F32_API int sgemm_f32_plan_ex(int layout, int transa, int transb, int64_t M, int64_t N,
                                    int64_t K, float alpha, const float *A, int64_t lda,
                                    const float *B, int64_t ldb, float beta, const float *C,
                                    int64_t ldc, int num_cus, int *variant);

/* Stream-K with a caller-owned workspace. The pages split only the tiles
 * that would form the last, partially filled round of the compute units
 * along K, and combine the partial sums of each such tile ("Optimizing
 * Matrix Multiply on CUDA, Part 2", "Distributing the Partially Filled
 * Wave"). Here: with T tiles on C compute units, floor(T/C)*C tiles are
 * computed whole; the other T mod C tiles' K slices are dealt out in equal
 * runs to at most min(C, 4*(T mod C)) workgroups (a tile is cut into about
 * four pieces at most, as the pages found best). A run that covers a whole
 * tile writes C; the others write their partial tiles to the workspace, and
 * a second kernel on the same stream sums each split tile's pieces in K
 * order -- so results are deterministic for a given device and shape -- and
 * applies alpha and beta. (The pages combine the pieces in the unit that
 * finishes a tile's last piece; on MI355X the device-scope fences that
 * needs write back or invalidate a whole XCD's L2 per piece, which costs
 * more than the second launch.) No workgroup waits for another.
 *
 * sgemm_f32_ws is sgemm_f32_ex with a workspace: the automatic choice may
 * then also pick a stream-K kernel (SGEMM_F32_MFMA_128_SK,
 * SGEMM_F32_MFMA_64x128_SK, SGEMM_F32_MFMA_256_SK) when the dispatch model predicts it faster and
 * `workspace_bytes` covers what it needs. With workspace_bytes == 0 (the
 * workspace may then be NULL) it is sgemm_f32_ex. The workspace is device
 * memory of at least workspace_bytes bytes, 16-byte aligned, owned by the
 * caller; its contents on entry do not matter, and on return they are
 * undefined. Calls that may run at the same time (different streams) need
 * different workspaces. */
SGEMM_F32_API int sgemm_f32_ws(int layout, int transa, int transb, int64_t M, int64_t N, int64_t K,
                               float alpha, const float *A, int64_t lda, const float *B,
                               int64_t ldb, float beta, float *C, int64_t ldc, void *workspace,
                               size_t workspace_bytes, void *stream);

/* sgemm_f32_ws with the kernel forced to `variant`. A stream-K variant given
 * less workspace than it needs returns SGEMM_F32_ERR_WORKSPACE; on a shape
 * that it does not split (T a multiple of C) it needs none and runs as its
 * whole-tile kernel. Other variants ignore the workspace. sgemm_f32_variant
 * and sgemm_f32_variant_ex pass no workspace. */
SGEMM_F32_API int sgemm_f32_variant_ws(int variant, int layout, int transa, int transb, int64_t M,
                                       int64_t N, int64_t K, float alpha, const float *A,
                                       int64_t lda, const float *B, int64_t ldb, float beta,
                                       float *C, int64_t ldc, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * stream-K entry points with the library's own fixed scratch as the
 * workspace, so that nothing is allocated, on the call path or before it.
 * variant == -1 is sgemm_f32_ws with workspace_bytes =
 * SGEMM_F32_SCRATCH_BYTES: the automatic choice, whose stream-K candidates
 * are only those whose workspace fits the scratch. variant >= 0 is
 * sgemm_f32_variant_ws with that workspace; a stream-K variant that would
 * need more than SGEMM_F32_SCRATCH_BYTES on this problem returns
 * SGEMM_F32_ERR_SCRATCH before anything is launched. Arguments, ownership of
 * A, B and C, asynchrony and the other return codes are those of
 * sgemm_f32_ws / sgemm_f32_variant_ws; SGEMM_F32_ERR_VARIANT for variant < -1.
 *
 * The scratch is one file-scope device array per GPU, held from the library's
 * first use on that GPU until the process ends; its address is looked up
 * once per device (hipGetSymbolAddress, no allocation) on the first call with
 * that device current. Every call on one GPU shares it and it keeps the last
 * call's contents (the kernels never read what they have not written in the
 * same call, so nothing is cleared). Calls on one GPU whose executions can
 * overlap -- different streams without an ordering between them -- race on
 * the scratch and may return wrong results: order them, or use sgemm_f32_ws
 * with one workspace per stream. Calls on the same stream are ordered. */
SGEMM_F32_API int sgemm_f32_ws_static(int variant, int layout, int transa, int transb, int64_t M,
                                      int64_t N, int64_t K, float alpha, const float *A,
                                      int64_t lda, const float *B, int64_t ldb, float beta,
                                      float *C, int64_t ldc, void *stream);

/* The variant sgemm_f32_ws would launch with `workspace_bytes` of workspace,
 * as sgemm_f32_plan (host-only). */
SGEMM_F32_API int sgemm_f32_plan_ws(int layout, int transa, int transb, int64_t M, int64_t N,
                                    int64_t K, float alpha, const float *A, int64_t lda,
                                    const float *B, int64_t ldb, float beta, const float *C,
                                    int64_t ldc, size_t workspace_bytes, int num_cus,
                                    int *variant);

/* Workspace bytes that stream-K `variant` needs for this problem on a device
 * with num_cus compute units (0 if it would not split it, or if the variant
 * is not a stream-K kernel); with variant == -1, the most any stream-K
 * kernel the automatic choice may consider needs, so that passing that much
 * to sgemm_f32_ws leaves every candidate open. Host-only. Writes *bytes and
 * returns 0, or -13/-14/-15/-1/-2/-3 for a bad layout, flag or size, -12 if
 * bytes is NULL, SGEMM_F32_ERR_VARIANT, or SGEMM_F32_ERR_TOO_LARGE. At most
 * 2 * num_cus partial tiles of the kernel's block tile: 134 MB for the
 * 256 x 256 tiles on 256 compute units, 33.6 MB for 128 x 128. */
SGEMM_F32_API int sgemm_f32_ws_size(int variant, int layout, int transa, int transb, int64_t M,
                                    int64_t N, int64_t K, int num_cus, size_t *bytes);

/* 1 if `variant` reads transposed operands (mfma_128x128, mfma_256x256,
 * mfma_64x128, mfma_64x64, the K-group kernels, the stream-K kernels,
 * mfma_skinny and mfma_direct), 0 if not, or SGEMM_F32_ERR_VARIANT. */
SGEMM_F32_API int sgemm_f32_variant_trans_ok(int variant);

/* Geometry of a matrix-core tile kernel, the variants the dispatch model
 * (below) chooses among: *bm x *bn is the block of C one workgroup
 * computes, *bk the K depth of one step of its K loop, which is also the
 * unit in which a stream-K kernel splits K (sgemm_f32_ws_size). These are
 * compile-time parameters of the library, so a tuner reads them here rather
 * than assuming them. Host-only. Returns 1 and writes the non-NULL pointers
 * for a tile kernel; 0, writing zeros, for any other variant;
 * SGEMM_F32_ERR_VARIANT for an id out of range. */
SGEMM_F32_API int sgemm_f32_variant_tile(int variant, int *bm, int *bn, int *bk);

/* The dispatch model sgemm_f32 uses to choose among the tiled matrix-core
 * kernels (sgemm_f32_plan reports the choice). It follows the pages' kernel
 * selection by the busiest SM's work ("Optimizing Matrix Multiply on CUDA,
 * Part 2", "Selecting Among Three Kernels"), with measured constants: for a
 * candidate with block tile BM x BN on a device with C compute units, the
 * predicted time in microseconds is
 *     overhead_us + ceil(n) * tile_us + 1e6 * n * 2*BM*BN*K / (614.4e9 * eff[b] * f),
 * n = ceil(ceil(M/BM) * ceil(N/BN) / C), b = 0, 1, 2, 3 for n = 1, 2, 3-4, >= 5
 * (614.4e9 FLOP/s is one compute unit's FP32 matrix peak), f = 1 when both
 * operands can be filled with 16-byte loads and f = fill4 when not (a
 * leading dimension, the contiguous extent of an operand or a base address
 * that is not a whole number of 16-byte chunks: the kernels then load 4
 * bytes per lane, several times as many loads per slice). The smallest
 * prediction wins; ties go to the earlier entry. For a stream-K entry n is
 * the busiest unit's share, floor(T/C) whole tiles plus one run of slices
 * (a fraction of a tile), with b taken for ceil(n); stream-K entries are
 * considered only by sgemm_f32_ws, on shapes they split, and when the
 * workspace suffices; if no entry applies, mfma_128x128 runs. M <= 32 and
 * products of fewer than 64 Mi multiply-adds bypass the model (mfma_skinny,
 * mfma_direct; both read transposed operands); mfma_direct is also a model
 * entry for larger products. Otherwise a call with a transposed operand (after
 * the column-major swap) is restricted to the model's entries that read
 * transposed operands (mfma_128x128 if there are none). */
#define SGEMM_F32_MODEL_MAX 16
typedef struct {
    int variant;        /* a tiled matrix-core variant: MFMA_128, MFMA_256, MFMA_64x128, MFMA_64,
                           MFMA_64x128_KG4, MFMA_64x96_KG4, MFMA_96x64_KG4, MFMA_128x128_KG4,
                           MFMA_128_SK, MFMA_64x128_SK, MFMA_256_SK or MFMA_DIRECT (32x32
                           tiles, no LDS tile: its K split is inside the workgroup) */
    double overhead_us; /* fixed cost per call, microseconds, in [0, 1e6] */
    double eff[4];      /* fraction of peak per tiles-per-CU bucket, in (0, 1.5] */
    double fill4;       /* factor on eff for calls that need the 4-byte fill, in (0, 1.5] */
    double tile_us;     /* fixed cost per tile (or stream-K run) on the busiest unit, in
                           [0, 1e4] microseconds: a tile's first fill and its epilogue */
} sgemm_f32_model_entry;

/* Replace the process-wide dispatch model by entries[0..n). n = 0 restores the
 * built-in model (entries may then be NULL). The library copies the entries.
 * Returns 0; -1 if entries is NULL with n > 0; -2 if n is outside
 * [0, SGEMM_F32_MODEL_MAX]; -3 if an entry names a variant that is not a tiled
 * kernel, repeats one, or holds a value out of range (the model is then left
 * unchanged); -4 if host memory runs out. Safe to call while other threads
 * launch: each call sees either the old or the new model; each replacement
 * keeps about 1 KB of host memory until the process ends.
 * fp32_gemm_tuning_amd.tune fits a model to the current device. */
SGEMM_F32_API int sgemm_f32_set_model(const sgemm_f32_model_entry *entries, int n);

/* Copy the active model into out[0..cap). Returns the number of entries in the
 * model (which may exceed cap), or -1 if cap < 0 or out is NULL with cap > 0. */
SGEMM_F32_API int sgemm_f32_get_model(sgemm_f32_model_entry *out, int cap);

/* Number of variants (SGEMM_F32_NUM_VARIANTS). */
SGEMM_F32_API int sgemm_f32_num_variants(void);

/* Short name of a variant ("naive", ..., "mfma_64x128"), or NULL if out of range.
 * The string is static. */
SGEMM_F32_API const char *sgemm_f32_variant_name(int variant);

/* Variant id for a name, or -1. */
SGEMM_F32_API int sgemm_f32_variant_by_name(const char *name);

/* Static description of a return code. Never NULL. */
SGEMM_F32_API const char *sgemm_f32_strerror(int code);

/* Launch shape of a variant's main kernel on the current device, as the
 * pages print it before timing (Day 44, "Five paths, one table": registers,
 * spills, resident blocks): workgroup size, static LDS bytes, registers per
 * lane as the runtime reports them, scratch (spill) bytes per lane and the
 * number of workgroups resident per compute unit. Any output pointer may be
 * NULL. Returns 0, SGEMM_F32_ERR_VARIANT, SGEMM_F32_ERR_DEVICE or a positive
 * hipError_t. */
SGEMM_F32_API int sgemm_f32_kernel_info(int variant, int *threads, int *lds_bytes, int *regs,
                                        int *scratch_bytes, int *wg_per_cu);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_F32_H */
