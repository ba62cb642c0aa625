/*
 * CPU oracle for FP32 SGEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library. The product path (the HIP library) never calls it,
 * and the two share no code.
 *
 * What it computes is the plain definition of the product:
 *   C[i][j] = alpha * sum_k A[i][k] * B[k][j] + beta * C0[i][j]
 * with row-major operands, as written in "GEMM from scratch", Module 02
 * ("One Thread Per Output": each output is the K-term dot product of row i
 * of A and column j of B, scaled by alpha, plus beta times the old C), and as
 * counted in "Optimizing Matrix Multiply on CUDA, Part 1", section
 * "Counting the Work". "100 Days of GPU, Day 44", section "Five paths, one
 * table", checks every kernel against a double-precision CPU reference at
 * every element; this is that reference.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *  - Leading dimensions: element (i,k) of A is A[i*lda+k], (k,j) of B is
 *    B[k*ldb+j], (i,j) of C0 is C0[i*ldc+j]; the pages use packed strides.
 *  - beta == 0: C0 is not read (so an uninitialised C cannot inject NaN).
 *  - alpha == 0 or K == 0: A and B are not read; the result is beta*C0.
 *  - Arithmetic: every FP32 product is formed exactly in double (24+24 <= 53
 *    significant bits); the K products of one output are summed in double in
 *    ascending k order; no contraction (built with -ffp-contract=off).
 *  - Alongside each value the oracle returns the magnitude sum
 *      Babs[i][j] = |alpha| * sum_k |A[i][k] * B[k][j]| + |beta| * |C0[i][j]|
 *    which scales the elementwise error bound the tests apply.
 *
 * Loop order: rows in parallel (OpenMP), then k, then j, with one double
 * accumulator per output column; for a fixed output the k order is the same
 * ascending order as the textbook i-j-k triple loop.
 *
 * Return value: 0 on success, -1 if an argument is out of range (negative
 * size, leading dimension too small, missing pointer), -2 if scratch memory
 * could not be allocated.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int check_args(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                      int64_t lda, const float *B, int64_t ldb, float beta,
                      const float *C0, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1)) return -1;
    int reads_ab = (alpha != 0.0f) && K > 0 && M > 0 && N > 0;
    if (reads_ab && (A == NULL || B == NULL)) return -1;
    if (beta != 0.0f && M > 0 && N > 0 && C0 == NULL) return -1;
    return 0;
}

/* One output row i restricted to the column list cols[0..ncols) (or all
 * columns when cols == NULL). s and a are ncols-long double scratch rows. */
static void one_row(int64_t i, int64_t N, int64_t K, float alpha, const float *A,
                    int64_t lda, const float *B, int64_t ldb, float beta,
                    const float *C0, int64_t ldc, int64_t ncols, const int64_t *cols,
                    double *s, double *a, double *out, double *babs) {
    int64_t n = cols ? ncols : N;
    for (int64_t jj = 0; jj < n; ++jj) { s[jj] = 0.0; a[jj] = 0.0; }
    if (alpha != 0.0f) {
        for (int64_t k = 0; k < K; ++k) {
            double aik = (double)A[i * lda + k];
            const float *brow = B + k * ldb;
            if (cols) {
                for (int64_t jj = 0; jj < n; ++jj) {
                    double p = aik * (double)brow[cols[jj]];
                    s[jj] += p;
                    a[jj] += fabs(p);
                }
            } else {
                for (int64_t jj = 0; jj < n; ++jj) {
                    double p = aik * (double)brow[jj];
                    s[jj] += p;
                    a[jj] += fabs(p);
                }
            }
        }
    }
    double al = (double)alpha, be = (double)beta;
    for (int64_t jj = 0; jj < n; ++jj) {
        int64_t j = cols ? cols[jj] : jj;
        double v = al * s[jj];
        double m = fabs(al) * a[jj];
        if (beta != 0.0f) {
            double c = (double)C0[i * ldc + j];
            v += be * c;
            m += fabs(be) * fabs(c);
        }
        out[jj] = v;
        if (babs) babs[jj] = m;
    }
}

static int run(int64_t M, int64_t N, int64_t K, float alpha, const float *A, int64_t lda,
               const float *B, int64_t ldb, float beta, const float *C0, int64_t ldc,
               int64_t nrows, const int64_t *rows, int64_t ncols, const int64_t *cols,
               double *out, double *babs) {
    /* rows == NULL selects every row, cols == NULL every column. */
    int rc = check_args(M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc);
    if (rc) return rc;
    int64_t nr = rows ? nrows : M;
    int64_t nc = cols ? ncols : N;
    if (nr < 0 || nc < 0) return -1;
    if (nr > 0 && nc > 0 && out == NULL) return -1;
    for (int64_t r = 0; rows && r < nr; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    for (int64_t c = 0; cols && c < nc; ++c)
        if (cols[c] < 0 || cols[c] >= N) return -1;
    if (nr == 0 || nc == 0) return 0;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)nc);
        double *a = (double *)malloc(sizeof(double) * (size_t)nc);
        if (!s || !a) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < nr; ++r) {
            if (!s || !a) continue;
            int64_t i = rows ? rows[r] : r;
            one_row(i, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, nc, cols, s, a,
                    out + r * nc, babs ? babs + r * nc : NULL);
        }
        free(s);
        free(a);
    }
    return failed ? -2 : 0;
}

/* Every output: out and babs are M x N, packed row-major (leading dim N). */
int oracle_sgemm_f64(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                     int64_t lda, const float *B, int64_t ldb, float beta,
                     const float *C0, int64_t ldc, double *out, double *babs) {
    return run(M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, 0, NULL, 0, NULL, out, babs);
}

/* The listed rows only: out and babs are nrows x N, packed. */
int oracle_sgemm_f64_rows(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                          int64_t lda, const float *B, int64_t ldb, float beta,
                          const float *C0, int64_t ldc, int64_t nrows, const int64_t *rows,
                          double *out, double *babs) {
    if (nrows < 0 || (nrows > 0 && !rows)) return -1;
    if (nrows == 0) return check_args(M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc);
    return run(M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, nrows, rows, 0, NULL, out, babs);
}

/* The listed columns only: out and babs are M x ncols, packed. */
int oracle_sgemm_f64_cols(int64_t M, int64_t N, int64_t K, float alpha, const float *A,
                          int64_t lda, const float *B, int64_t ldb, float beta,
                          const float *C0, int64_t ldc, int64_t ncols, const int64_t *cols,
                          double *out, double *babs) {
    if (ncols < 0 || (ncols > 0 && !cols)) return -1;
    if (ncols == 0) return check_args(M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc);
    return run(M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, 0, NULL, ncols, cols, out, babs);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
