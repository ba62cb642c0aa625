// C-ABI entry points of libsgemm_f32: argument checks, quick returns, the
// host-side choice of kernel variant, and the launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <new>
#include <cstdlib>
#include <cstring>

#include "kernels.hpp"
#include "sgemm_f32.h"

namespace sgemm {

static const Variant* const kTable[SGEMM_F32_NUM_VARIANTS] = {
    &kNaive, &kCoalesced, &kLdsTiled, &kReg1d, &kReg2d, &kVec4TransA,
    &kValuMain, &kMfma128, &kMfma64, &kMfmaSkinny, &kMfmaKsplit, &kMfmaDirect, &kMfma64x128,
    &kMfma256, &kMfmaKgroup, &kMfmaKgroup96, &kMfmaKgroup128, &kMfma128Sk, &kMfma64x128Sk,
    &kMfma256Sk, &kMfmaKgroup96x64,
};

static bool misaligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; }
static bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
static int64_t max1(int64_t v) { return v > 1 ? v : 1; }

// Argument checks in signature order; returns the code of the first bad
// argument: -13 layout, -14 transa, -15 transb, then -1 M, -2 N, -3 K, -5 A,
// -6 lda, -7 B, -8 ldb, -10 C, -11 ldc (the positions of these arguments in
// sgemm_f32, counting M as 1). A and B must be valid only when they are read
// (M, N, K > 0 and alpha != 0); C only when it is written (M, N > 0). A
// leading dimension must cover the contiguous extent of its matrix as stored:
// for row-major storage the column count of the stored matrix (A stored
// M x K, or K x M when transposed), for column-major storage its row count.
static int validate(int layout, int transa, int transb, int64_t M, int64_t N, int64_t K,
                    float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                    const float* C, int64_t ldc) {
    if (layout != SGEMM_F32_ROW_MAJOR && layout != SGEMM_F32_COL_MAJOR) return -13;
    if (transa != SGEMM_F32_NO_TRANS && transa != SGEMM_F32_TRANS) return -14;
    if (transb != SGEMM_F32_NO_TRANS && transb != SGEMM_F32_TRANS) return -15;
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const bool col = layout == SGEMM_F32_COL_MAJOR;
    const int64_t a_contig = col ? (transa ? K : M) : (transa ? M : K);
    const int64_t b_contig = col ? (transb ? N : K) : (transb ? K : N);
    const int64_t c_contig = col ? M : N;
    const bool reads_ab = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
    const bool writes_c = M > 0 && N > 0;
    if (reads_ab && (A == nullptr || misaligned4(A))) return -5;
    if (lda < max1(a_contig)) return -6;
    if (reads_ab && (B == nullptr || misaligned4(B))) return -7;
    if (ldb < max1(b_contig)) return -8;
    if (writes_c && (C == nullptr || misaligned4(C))) return -10;
    if (ldc < max1(c_contig)) return -11;
    return 0;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Variant choice. Following the pages' tile selection ("Optimizing Matrix
// Multiply on CUDA, Part 2", "Selecting Among Three Kernels"; "Part 1",
// "Small and Odd Sizes"), the host predicts each candidate's time and takes
// the smallest. With T tiles dealt out to C compute units (MI355X places
// workgroups breadth-first), the busiest unit holds n = ceil(T / C) tiles;
// the prediction is a fixed cost (launch, first fill, epilogue) plus that
// unit's n * 2*BM*BN*K FLOP at a fraction of its peak that depends on n
// (few tiles per unit leave the matrix cores waiting on fills and barriers),
// times a per-kernel factor when the operand rows are not whole 16-byte
// chunks (register-staged or 4-byte fills), plus a fixed cost per tile on
// that unit (a tile's first fill and epilogue). All four were fitted per
// kernel to interleaved timings of every candidate on 30 shapes from 512^3
// to 8192^3, square, flat, tall and odd, on MI355X
// (fp32_gemm_tuning_amd/tune.py): in sample the model picks the fastest
// kernel on 27 of them (worst 2.3% lost). On 24 random shapes it was not
// fitted to (sides log-uniform in [300, 6000]) it picks the fastest
// whole-tile kernel on 18 without a workspace and the fastest of all on 20
// with one, losing 0.5% and 0.6% on average (worst 4.5% and 8.6%).
// ---------------------------------------------------------------------------
struct Candidate {
    int variant;
    double overhead_us;
    double eff[4];  // fraction of peak with n = 1, 2, 3-4, >= 5 tiles per CU
    double fill4;   // factor on eff when the operands need the 4-byte fill
    double tile_us; // fixed cost per tile (or stream-K run) on the busiest unit
};

// The variants the model can choose among: the matrix-core tile kernels,
// whose block tile and (for the stream-K kernels) K slice the variant table
// records.
static const int kModelVariants[] = {
    SGEMM_F32_MFMA_128,      SGEMM_F32_MFMA_256,       SGEMM_F32_MFMA_64x128,
    SGEMM_F32_MFMA_64,       SGEMM_F32_MFMA_64x128_KG4, SGEMM_F32_MFMA_64x96_KG4,
    SGEMM_F32_MFMA_96x64_KG4, SGEMM_F32_MFMA_128x128_KG4, SGEMM_F32_MFMA_128_SK, SGEMM_F32_MFMA_64x128_SK,
    SGEMM_F32_MFMA_256_SK,   SGEMM_F32_MFMA_DIRECT,
};
static bool model_variant(int variant) {
    for (int v : kModelVariants)
        if (v == variant) return true;
    return false;
}

static constexpr int kMaxModel = SGEMM_F32_MODEL_MAX;
struct Model {
    int n;
    Candidate c[kMaxModel];
};

// Built-in model, listed in order of preference when predictions tie.
static const Model kDefaultModel = {12,
                                    {
                                        {SGEMM_F32_MFMA_128, 0.0, {0.919, 0.949, 0.970, 0.967}, 0.88, 6.5},
                                        {SGEMM_F32_MFMA_256, 0.0, {0.993, 0.959, 0.976, 0.976}, 0.86, 13.0},
                                        {SGEMM_F32_MFMA_64x128, 0.5, {0.748, 0.838, 0.905, 0.922}, 0.78, 3.0},
                                        {SGEMM_F32_MFMA_64, 2.5, {0.703, 0.801, 0.822, 0.909}, 0.82, 1.5},
                                        {SGEMM_F32_MFMA_64x128_KG4, 1.5, {0.774, 0.784, 0.828, 0.861}, 0.96, 5.5},
                                        {SGEMM_F32_MFMA_64x96_KG4, 4.0, {0.748, 0.770, 0.756, 0.799}, 0.90, 4.5},
                                        {SGEMM_F32_MFMA_96x64_KG4, 3.5, {0.762, 0.785, 0.770, 0.814}, 0.94, 5.0},
                                        {SGEMM_F32_MFMA_128x128_KG4, 0.5, {0.910, 0.922, 0.943, 0.934}, 0.84, 10.0},
                                        {SGEMM_F32_MFMA_128_SK, 11.5, {0.794, 0.983, 0.967, 0.925}, 0.88, 4.5},
                                        {SGEMM_F32_MFMA_64x128_SK, 10.0, {0.720, 0.844, 1.000, 0.917}, 0.78, 2.5},
                                        {SGEMM_F32_MFMA_256_SK, 10.0, {0.961, 0.937, 0.977, 0.977}, 0.80, 20.0},
                                        // Fitted to per-launch timings around the tiny-product
                                        // bound: one 32x32 tile per compute unit fits 4.9 us +
                                        // 0.0087 us per k (eff 0.376), two tiles eff 0.40-0.44
                                        // (7 shapes); three or more are set low (measured
                                        // 0.30-0.43), where mfma_64x64 mostly wins.
                                        {SGEMM_F32_MFMA_DIRECT, 4.9, {0.376, 0.42, 0.35, 0.31}, 0.63, 0.0},
                                    }};
// The active model. A replacement is published by swapping this pointer;
// superseded models are never freed, so a concurrent reader never sees a
// model change under it (each replacement keeps about 1 KB).
static std::atomic<const Model*> g_model{&kDefaultModel};

// Peak FP32 FLOP/s of one compute unit: 4 SIMDs x 64 FLOP/clk x 2.4 GHz.
static const double kPeakPerCu = 4.0 * 64.0 * 2.4e9;
// At or below this many rows the skinny kernel (HBM-bound regime) is used.
static const int64_t kSkinnyMaxM = 32;
// Below this many multiply-adds launch latency dominates and the fine-tiled
// direct kernel is fastest (e.g. 256^3).
static const double kTinyMacs = 64.0 * 1024 * 1024;

static double eff_at(const Candidate& c, double n) {
    return n <= 1.0 ? c.eff[0] : n <= 2.0 ? c.eff[1] : n <= 4.0 ? c.eff[2] : c.eff[3];
}

// Tiles' worth of work on the busiest compute unit for a candidate: whole
// tiles dealt out breadth-first, or, for a stream-K kernel, the whole tiles
// plus one run of slices (sk_split). 0 if a stream-K kernel would not split.
static double busiest_tiles(const Variant& v, int64_t M, int64_t N, int64_t K, int num_cus) {
    const int64_t tiles = cdiv(M, v.bm) * cdiv(N, v.bn);
    if (v.ws_size != nullptr) {
        const SkSplit sp = sk_split(tiles, cdiv(K, v.bk), num_cus);
        return sp.split() ? sp.busiest_tiles(num_cus) : 0.0;
    }
    return (double)cdiv(tiles, num_cus);
}

// `trans`: an operand is stored transposed (after the column-major swap);
// only the kernels that read transposed operands are then candidates. A
// kernel whose instance for this call spills registers (Variant::auto_ok)
// is no candidate. The stream-K kernels are candidates only when they split
// this shape and `ws_bytes` covers the workspace they need. If no entry of
// the model applies, mfma_128x128 (which takes any shape, transposed or not,
// without spilling) runs.
static int choose(const Args& a, int num_cus, size_t ws_bytes) {
    if (num_cus < 1) num_cus = 1;
    const int64_t M = a.M, N = a.N, K = a.K;
    const bool trans = a.ta || a.tb;
    if (M <= kSkinnyMaxM) return SGEMM_F32_MFMA_SKINNY;
    if ((double)M * N * K < kTinyMacs) return SGEMM_F32_MFMA_DIRECT;
    const Model* m = g_model.load(std::memory_order_acquire);
    const bool vec = vec_ok(a);
    int best = SGEMM_F32_MFMA_128;
    double best_us = 0.0;
    bool found = false;
    for (int i = 0; i < m->n; ++i) {
        const Candidate& c = m->c[i];
        const Variant& v = *kTable[c.variant];
        if (trans && !v.trans_ok) continue;
        if (v.auto_ok != nullptr && !v.auto_ok(a)) continue;   // its instance would spill
        if (v.ws_size != nullptr && (ws_bytes == 0 || v.ws_size(a, num_cus) > ws_bytes)) continue;
        const double n = busiest_tiles(v, M, N, K, num_cus);
        if (n <= 0.0) continue;
        const double eff = eff_at(c, std::ceil(n)) * (vec ? 1.0 : c.fill4);
        const double us = c.overhead_us + std::ceil(n) * c.tile_us +
                          1e6 * n * 2.0 * v.bm * v.bn * (double)K / (kPeakPerCu * eff);
        if (!found || us < best_us) {
            best = c.variant;
            best_us = us;
            found = true;
        }
    }
    return best;
}

// ---------------------------------------------------------------------------
// Per-device compute-unit count, queried once per device.
// ---------------------------------------------------------------------------
static constexpr int kMaxDevices = 64;
static std::atomic<int> g_cus[kMaxDevices];

static int device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SGEMM_F32_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int cached = g_cus[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *cus = cached;
            return 0;
        }
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return SGEMM_F32_ERR_DEVICE;
    if (dev < kMaxDevices) g_cus[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return 0;
}

int xcd_remap_enabled() {
    static std::atomic<int> v{-1};
    int cur = v.load(std::memory_order_relaxed);
    if (cur < 0) {
        const char* e = getenv("SGEMM_F32_XCD_REMAP");
        cur = (e && e[0] == '0') ? 0 : 1;
        v.store(cur, std::memory_order_relaxed);
    }
    return cur;
}

// The row-major problem the kernels solve. A column-major call is the same
// product transposed: C^T = op(B)^T op(A)^T, where the column-major storage of
// each matrix is the row-major storage of its transpose. So the operands and
// M, N swap places, and so do the transposition flags. ("100 Days of GPU",
// Day 44, "Five paths, one table": the column-major library call with
// swapped operands yields the row-major product in place; this is the same
// identity used the other way round.)
static Args make_args(int layout, int transa, int transb, int64_t M, int64_t N, int64_t K,
                      float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                      float beta, float* C, int64_t ldc) {
    const bool col = layout == SGEMM_F32_COL_MAJOR;
    Args a;
    a.A = col ? B : A;
    a.B = col ? A : B;
    a.C = C;
    a.lda = col ? ldb : lda;
    a.ldb = col ? lda : ldb;
    a.ldc = ldc;
    a.M = (int32_t)(col ? N : M);
    a.N = (int32_t)(col ? M : N);
    a.K = (int32_t)K;
    a.alpha = alpha;
    a.beta = beta;
    a.ta = col ? transb : transa;
    a.tb = col ? transa : transb;
    a.tc = 0;
    return a;
}

// A product with few columns and more rows (a row-major call with N <= 32,
// or a column-major call with M <= 32, which the swap turns into one) is one
// no kernel serves well as it stands. Its transpose has few rows:
// C^T = op(B)^T op(A)^T, where op(B)^T is read through B with its
// transposition flag flipped, op(A)^T through A likewise, and C^T is C
// written column-major (Args::tc). The skinny kernel computes that.
// Returns the variant for the automatic choice, with `a` replaced by the
// transposed problem when that applies.
static int plan_args(const Args& a, int num_cus, size_t ws_bytes);
static int plan_call(Args& a, int num_cus, size_t ws_bytes) {
    if (a.N <= kSkinnyMaxM && a.M > kSkinnyMaxM) {
        Args u = a;
        u.A = a.B;
        u.B = a.A;
        u.lda = a.ldb;
        u.ldb = a.lda;
        u.M = a.N;
        u.N = a.M;
        u.ta = !a.tb;
        u.tb = !a.ta;
        u.tc = 1;
        if (kTable[SGEMM_F32_MFMA_SKINNY]->check(u) == 0) {
            a = u;
            return SGEMM_F32_MFMA_SKINNY;
        }
    }
    return plan_args(a, num_cus, ws_bytes);
}

// The variant the automatic choice launches for a (valid, non-quick-return)
// row-major problem. Shapes beyond a kernel's 32-bit buffer offsets fall back
// to the plain-pointer register-tiled rung, which reads untransposed
// operands only; a transposed call keeps its choice and fails its check.
static int plan_args(const Args& a, int num_cus, size_t ws_bytes) {
    const bool trans = a.ta || a.tb;
    int v = choose(a, num_cus, ws_bytes);
    if (!trans && kTable[v]->check(a) != 0) v = SGEMM_F32_REG_2D;
    return v;
}

// A workspace of nonzero size must be a 16-byte aligned device pointer.
static int validate_ws(const void* ws, size_t ws_bytes) {
    return (ws_bytes > 0 && (ws == nullptr || misaligned16(ws))) ? -16 : 0;
}

// `ws_short` is the code returned when a forced stream-K variant needs more
// workspace than `ws_bytes`.
static int run(int forced, int layout, int transa, int transb, int64_t M, int64_t N, int64_t K,
               float alpha, const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
               float* C, int64_t ldc, void* ws, size_t ws_bytes, void* stream,
               int ws_short = SGEMM_F32_ERR_WORKSPACE) {
    if (forced >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    int rc = validate(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (rc) return rc;
    rc = validate_ws(ws, ws_bytes);
    if (rc) return rc;
    if (M == 0 || N == 0) return 0;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return SGEMM_F32_ERR_TOO_LARGE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    Args a = make_args(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc);
    if (K == 0 || alpha == 0.0f) {
        const hipError_t e = launch_scale(a, s);
        return e == hipSuccess ? 0 : (int)e;
    }
    int v = forced, cus = 0;
    if (v < 0 || kTable[v]->launch_ws != nullptr) {
        rc = device_cus(&cus);
        if (rc) return rc;
    }
    if (v < 0) v = plan_call(a, cus, ws_bytes);
    const Variant& var = *kTable[v];
    if ((a.ta || a.tb) && !var.trans_ok) return SGEMM_F32_ERR_UNSUPPORTED;
    rc = var.check(a);
    if (rc) return rc;
    hipError_t e;
    if (var.launch_ws != nullptr) {
        if (var.ws_size(a, cus) > ws_bytes) return ws_short;
        e = var.launch_ws(a, ws, ws_bytes, cus, s);
    } else {
        e = var.launch(a, s);
    }
    return e == hipSuccess ? 0 : (int)e;
}

// ---------------------------------------------------------------------------
// Fixed device scratch for sgemm_f32_ws_static: the stream-K partial tiles of
// callers that cannot allocate. Each device the library runs on holds its own
// copy from the code object's load until the process ends. In host code the
// name `scratch` is only a stand-in for the symbol, never a device address:
// kernels get the address hipGetSymbolAddress returns for the current device.
// ---------------------------------------------------------------------------
static constexpr size_t kScratchBytes = SGEMM_F32_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static std::atomic<void*> g_scratch[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device (with
// that device current) and kept. Concurrent first calls may both look it up;
// they get the same address.
static int scratch_ptr(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return SGEMM_F32_ERR_DEVICE;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (p == nullptr) return SGEMM_F32_ERR_DEVICE;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return 0;
}

static int plan(int layout, int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                const float* A, int64_t lda, const float* B, int64_t ldb, float beta, const float* C,
                int64_t ldc, size_t ws_bytes, int num_cus, int* variant) {
    int rc = validate(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (rc) return rc;
    if (variant == nullptr) return -12;
    if (M == 0 || N == 0 || K == 0 || alpha == 0.0f) {
        *variant = -1;
        return 0;
    }
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return SGEMM_F32_ERR_TOO_LARGE;
    Args a = make_args(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta,
                       const_cast<float*>(C), ldc);
    *variant = plan_call(a, num_cus, ws_bytes);
    return 0;
}

// Workspace a stream-K variant (or, with variant == -1, the largest any of
// them) needs for this problem on num_cus compute units.
static int ws_size(int variant, int layout, int transa, int transb, int64_t M, int64_t N,
                   int64_t K, int num_cus, size_t* bytes) {
    if (variant < -1 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    if (layout != SGEMM_F32_ROW_MAJOR && layout != SGEMM_F32_COL_MAJOR) return -13;
    if (transa != SGEMM_F32_NO_TRANS && transa != SGEMM_F32_TRANS) return -14;
    if (transb != SGEMM_F32_NO_TRANS && transb != SGEMM_F32_TRANS) return -15;
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    if (bytes == nullptr) return -12;
    *bytes = 0;
    if (M == 0 || N == 0 || K == 0) return 0;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return SGEMM_F32_ERR_TOO_LARGE;
    if (num_cus < 1) num_cus = 1;
    // Only the sizes and flags matter for the workspace.
    const Args a = make_args(layout, transa, transb, M, N, K, 1.0f, nullptr, 1, nullptr, 1, 0.0f,
                             nullptr, 1);
    const bool trans = a.ta || a.tb;
    for (int v = 0; v < SGEMM_F32_NUM_VARIANTS; ++v) {
        const Variant& var = *kTable[v];
        if (var.ws_size == nullptr || (variant >= 0 && v != variant)) continue;
        if (variant < 0 && trans && !var.trans_ok) continue;
        const size_t need = var.ws_size(a, num_cus);
        if (need > *bytes) *bytes = need;
    }
    return 0;
}

}  // namespace sgemm

using namespace sgemm;

extern "C" {

SGEMM_F32_API int sgemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                            int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                            int64_t ldc, void* stream) {
    return run(-1, SGEMM_F32_ROW_MAJOR, SGEMM_F32_NO_TRANS, SGEMM_F32_NO_TRANS, M, N, K, alpha, A,
               lda, B, ldb, beta, C, ldc, nullptr, 0, stream);
}

SGEMM_F32_API int sgemm_f32_variant(int variant, int64_t M, int64_t N, int64_t K, float alpha,
                                    const float* A, int64_t lda, const float* B, int64_t ldb,
                                    float beta, float* C, int64_t ldc, void* stream) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    return run(variant, SGEMM_F32_ROW_MAJOR, SGEMM_F32_NO_TRANS, SGEMM_F32_NO_TRANS, M, N, K, alpha,
               A, lda, B, ldb, beta, C, ldc, nullptr, 0, stream);
}

SGEMM_F32_API int sgemm_f32_plan(int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                                 int64_t lda, const float* B, int64_t ldb, float beta,
                                 const float* C, int64_t ldc, int num_cus, int* variant) {
    return plan(SGEMM_F32_ROW_MAJOR, SGEMM_F32_NO_TRANS, SGEMM_F32_NO_TRANS, M, N, K, alpha, A, lda,
                B, ldb, beta, C, ldc, 0, num_cus, variant);
}

SGEMM_F32_API int sgemm_f32_ex(int layout, int transa, int transb, int64_t M, int64_t N, int64_t K,
                               float alpha, const float* A, int64_t lda, const float* B,
                               int64_t ldb, float beta, float* C, int64_t ldc, void* stream) {
    return run(-1, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, nullptr, 0,
               stream);
}

SGEMM_F32_API int sgemm_f32_variant_ex(int variant, int layout, int transa, int transb, int64_t M,
                                       int64_t N, int64_t K, float alpha, const float* A,
                                       int64_t lda, const float* B, int64_t ldb, float beta,
                                       float* C, int64_t ldc, void* stream) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    return run(variant, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               nullptr, 0, stream);
}

SGEMM_F32_API int sgemm_f32_plan_ex(int layout, int transa, int transb, int64_t M, int64_t N,
                                    int64_t K, float alpha, const float* A, int64_t lda,
                                    const float* B, int64_t ldb, float beta, const float* C,
                                    int64_t ldc, int num_cus, int* variant) {
    return plan(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, 0, num_cus,
                variant);
}

SGEMM_F32_API int sgemm_f32_ws(int layout, int transa, int transb, int64_t M, int64_t N, int64_t K,
                               float alpha, const float* A, int64_t lda, const float* B,
                               int64_t ldb, float beta, float* C, int64_t ldc, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return run(-1, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
               workspace_bytes, stream);
}

SGEMM_F32_API int sgemm_f32_variant_ws(int variant, int layout, int transa, int transb, int64_t M,
                                       int64_t N, int64_t K, float alpha, const float* A,
                                       int64_t lda, const float* B, int64_t ldb, float beta,
                                       float* C, int64_t ldc, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    return run(variant, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               workspace, workspace_bytes, stream);
}

SGEMM_F32_API int sgemm_f32_ws_static(int variant, int layout, int transa, int transb, int64_t M,
                                      int64_t N, int64_t K, float alpha, const float* A,
                                      int64_t lda, const float* B, int64_t ldb, float beta,
                                      float* C, int64_t ldc, void* stream) {
    if (variant < -1 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    // Argument errors and the empty product are reported before any HIP call.
    int rc = validate(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (rc) return rc;
    if (M == 0 || N == 0) return 0;
    void* ws = nullptr;
    rc = scratch_ptr(&ws);
    if (rc) return rc;
    return run(variant, layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws,
               kScratchBytes, stream, SGEMM_F32_ERR_SCRATCH);
}

SGEMM_F32_API int sgemm_f32_plan_ws(int layout, int transa, int transb, int64_t M, int64_t N,
                                    int64_t K, float alpha, const float* A, int64_t lda,
                                    const float* B, int64_t ldb, float beta, const float* C,
                                    int64_t ldc, size_t workspace_bytes, int num_cus,
                                    int* variant) {
    return plan(layout, transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                workspace_bytes, num_cus, variant);
}

SGEMM_F32_API int sgemm_f32_ws_size(int variant, int layout, int transa, int transb, int64_t M,
                                    int64_t N, int64_t K, int num_cus, size_t* bytes) {
    return ws_size(variant, layout, transa, transb, M, N, K, num_cus, bytes);
}

SGEMM_F32_API int sgemm_f32_variant_trans_ok(int variant) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    return kTable[variant]->trans_ok ? 1 : 0;
}

SGEMM_F32_API int sgemm_f32_variant_tile(int variant, int* bm, int* bn, int* bk) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    const bool tile = model_variant(variant);
    const Variant& v = *kTable[variant];
    if (bm != nullptr) *bm = tile ? v.bm : 0;
    if (bn != nullptr) *bn = tile ? v.bn : 0;
    if (bk != nullptr) *bk = tile ? v.bk : 0;
    return tile ? 1 : 0;
}

SGEMM_F32_API int sgemm_f32_num_variants(void) { return SGEMM_F32_NUM_VARIANTS; }

SGEMM_F32_API const char* sgemm_f32_variant_name(int variant) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return nullptr;
    return kTable[variant]->name;
}

SGEMM_F32_API int sgemm_f32_variant_by_name(const char* name) {
    if (name == nullptr) return -1;
    for (int i = 0; i < SGEMM_F32_NUM_VARIANTS; ++i)
        if (std::strcmp(kTable[i]->name, name) == 0) return i;
    return -1;
}

SGEMM_F32_API const char* sgemm_f32_strerror(int code) {
    switch (code) {
        case 0: return "success";
        case -1: return "argument 1 (M) is negative";
        case -2: return "argument 2 (N) is negative";
        case -3: return "argument 3 (K) is negative";
        case -5: return "argument 5 (A) is NULL or not 4-byte aligned";
        case -6: return "argument 6 (lda) is smaller than the contiguous extent of A as stored "
                        "(max(1, K) for row-major, untransposed A)";
        case -7: return "argument 7 (B) is NULL or not 4-byte aligned";
        case -8: return "argument 8 (ldb) is smaller than the contiguous extent of B as stored "
                        "(max(1, N) for row-major, untransposed B)";
        case -10: return "argument 10 (C) is NULL or not 4-byte aligned";
        case -11: return "argument 11 (ldc) is smaller than the contiguous extent of C "
                         "(max(1, N) row-major, max(1, M) column-major)";
        case -12: return "output pointer is NULL";
        case -13: return "layout is neither SGEMM_F32_ROW_MAJOR nor SGEMM_F32_COL_MAJOR";
        case -14: return "transa is neither SGEMM_F32_NO_TRANS nor SGEMM_F32_TRANS";
        case -15: return "transb is neither SGEMM_F32_NO_TRANS nor SGEMM_F32_TRANS";
        case -16: return "workspace is NULL with a nonzero size, or not 16-byte aligned";
        case SGEMM_F32_ERR_WORKSPACE: return "the stream-K variant needs a larger workspace (sgemm_f32_ws_size)";
        case SGEMM_F32_ERR_SCRATCH: return "the stream-K variant needs more workspace than the "
                                           "library's fixed scratch holds (SGEMM_F32_SCRATCH_BYTES)";
        case SGEMM_F32_ERR_VARIANT: return "variant id out of range";
        case SGEMM_F32_ERR_UNSUPPORTED: return "variant cannot run this shape, alignment or transposition";
        case SGEMM_F32_ERR_TOO_LARGE: return "a size exceeds what the kernel can index";
        case SGEMM_F32_ERR_DEVICE: return "no usable HIP device";
        default: break;
    }
    if (code > 0) return hipGetErrorString((hipError_t)code);
    return "unknown error";
}

SGEMM_F32_API int sgemm_f32_kernel_info(int variant, int* threads, int* lds_bytes, int* regs,
                                        int* scratch_bytes, int* wg_per_cu) {
    if (variant < 0 || variant >= SGEMM_F32_NUM_VARIANTS) return SGEMM_F32_ERR_VARIANT;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SGEMM_F32_ERR_DEVICE;
    const Variant& v = *kTable[variant];
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, v.kernel);
    if (e != hipSuccess) return (int)e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, v.kernel, v.threads, 0);
    if (e != hipSuccess) return (int)e;
    if (threads) *threads = v.threads;
    if (lds_bytes) *lds_bytes = (int)attr.sharedSizeBytes;
    if (regs) *regs = attr.numRegs;
    if (scratch_bytes) *scratch_bytes = (int)attr.localSizeBytes;
    if (wg_per_cu) *wg_per_cu = occ;
    return 0;
}

}  // extern "C"

extern "C" SGEMM_F32_API int sgemm_f32_set_model(const sgemm_f32_model_entry* entries, int n) {
    if (n < 0 || n > kMaxModel) return -2;
    if (n == 0) {
        g_model.store(&kDefaultModel, std::memory_order_release);
        return 0;
    }
    if (entries == nullptr) return -1;
    Model* m = new (std::nothrow) Model();
    if (m == nullptr) return -4;
    m->n = n;
    for (int i = 0; i < n; ++i) {
        const sgemm_f32_model_entry& e = entries[i];
        bool ok = model_variant(e.variant) && e.overhead_us >= 0.0 && e.overhead_us <= 1e6 &&
                  e.fill4 > 0.0 && e.fill4 <= 1.5 && e.tile_us >= 0.0 && e.tile_us <= 1e4;
        for (int b = 0; b < 4; ++b) ok = ok && e.eff[b] > 0.0 && e.eff[b] <= 1.5;
        for (int p = 0; p < i; ++p) ok = ok && entries[p].variant != e.variant;
        if (!ok) {
            delete m;
            return -3;
        }
        m->c[i] = Candidate{e.variant, e.overhead_us, {e.eff[0], e.eff[1], e.eff[2], e.eff[3]},
                            e.fill4, e.tile_us};
    }
    g_model.store(m, std::memory_order_release);
    return 0;
}

extern "C" SGEMM_F32_API int sgemm_f32_get_model(sgemm_f32_model_entry* out, int cap) {
    if (cap < 0 || (out == nullptr && cap > 0)) return -1;
    const Model* m = g_model.load(std::memory_order_acquire);
    for (int i = 0; i < m->n && i < cap; ++i) {
        const Candidate& c = m->c[i];
        out[i].variant = c.variant;
        out[i].overhead_us = c.overhead_us;
        for (int b = 0; b < 4; ++b) out[i].eff[b] = c.eff[b];
        out[i].fill4 = c.fill4;
        out[i].tile_us = c.tile_us;
    }
    return m->n;
}
