"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes the oracle to something independent: a hand-worked example,
closed forms (identity, permutation, all-ones, rank one), exact integer
arithmetic, exact rational arithmetic on tiny shapes, a library routine on a
special case, and the algebraic identities the definition implies
(linearity in alpha and beta, (AB)^T = B^T A^T). Definition pinned:
C = alpha*A*B + beta*C0, row-major ("GEMM from scratch", Module 02, "One
Thread Per Output"; "Optimizing Matrix Multiply on CUDA, Part 1", "Counting
the Work").

Setting ORACLE_LIB to another build of oracle.c runs these same pins against
it; tests/test_oracle_mutants.py uses that to check that planted mistakes are
caught.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from datagen import draw, draw_matrix


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U_D = 2.0 ** -53


@pytest.fixture(scope="module")
def lib():
    path = os.environ.get("ORACLE_LIB")
    if path:
        return oracle.open_lib(path)
    oracle.build(force=False)
    return oracle.open_lib(oracle.lib_path())


def ref(lib, A, B, C0=None, alpha=1.0, beta=0.0, **kw):
    return oracle.sgemm_ref(A, B, C0, alpha, beta, lib=lib, **kw)


def rng_mat(seed, r, c, dist="uniform"):
    return draw(np.random.default_rng(seed), (r, c), dist)


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(":")
            vals[key.strip()] = [float(x) for x in rest.split()]
    return vals


def test_hand_worked_example(lib):
    g = _read_golden("hand_example_2x3x2.txt")
    M, N, K = (int(x) for x in g["M N K"])
    A = np.array(g["A"], np.float32).reshape(M, K)
    B = np.array(g["B"], np.float32).reshape(K, N)
    C0 = np.array(g["C0"], np.float32).reshape(M, N)
    C, babs = ref(lib, A, B, C0, g["alpha"][0], g["beta"][0])
    assert np.array_equal(C, np.array(g["C"]).reshape(M, N))
    # |alpha|*(|A||B|) + |beta|*|C0| with all-positive A and B: 2*AB + |C0|
    assert np.array_equal(babs, np.array([[117, 130], [281, 312]], np.float64))


def test_identity_exact(lib):
    # A = I: C = alpha*B + beta*C0 exactly. B and C0 sit in wider buffers whose
    # padding columns are NaN, so a wrong leading dimension shows up.
    K, N = 37, 29
    A = np.eye(K, dtype=np.float32)
    Bbuf = draw_matrix(5, K, N, "uniform", ld=N + 7)
    C0buf = draw_matrix(6, K, N, "uniform", ld=N + 3)
    B, C0 = Bbuf[:, :N], C0buf[:, :N]
    C, _ = ref(lib, A, B)
    assert np.array_equal(C, B.astype(np.float64))
    C, _ = ref(lib, A, B, C0, 2.0, 0.5)
    assert np.array_equal(C, 2.0 * B.astype(np.float64) + 0.5 * C0.astype(np.float64))


def test_permutation_exact(lib):
    rng = np.random.default_rng(7)
    M = K = 41
    N = 23
    perm = rng.permutation(M)
    P = np.zeros((M, K), np.float32)
    P[np.arange(M), perm] = 1.0
    B = rng_mat(8, K, N)
    C, _ = ref(lib, P, B)
    assert np.array_equal(C, B[perm].astype(np.float64))
    # a permutation on the right permutes columns of A
    A = rng_mat(9, 19, K)
    Q = np.zeros((K, K), np.float32)
    q = rng.permutation(K)
    Q[q, np.arange(K)] = 1.0          # (A Q)[:, j] = A[:, q[j]]
    C, _ = ref(lib, A, Q)
    assert np.array_equal(C, A[:, q].astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 9, 300), (64, 64, 1000)])
def test_all_ones(lib, M, N, K):
    C, babs = ref(lib, np.ones((M, K), np.float32), np.ones((K, N), np.float32))
    assert np.all(C == K) and np.all(babs == K)


def test_rank_one_integer(lib):
    rng = np.random.default_rng(10)
    M, N, K = 13, 11, 257
    a = rng.integers(-3, 4, size=M).astype(np.float32)
    b = rng.integers(-3, 4, size=N).astype(np.float32)
    A = np.repeat(a[:, None], K, axis=1)
    B = np.repeat(b[None, :], K, axis=0)
    C, _ = ref(lib, A, B)
    assert np.array_equal(C, K * np.outer(a, b).astype(np.float64))


def test_small_integers_match_exact_int64(lib):
    # {-3..3} entries: every partial sum is an integer, so the result is exact;
    # compare with exact 64-bit integer arithmetic.
    rng = np.random.default_rng(11)
    M, N, K = 70, 50, 400
    A = rng.integers(-3, 4, size=(M, K))
    B = rng.integers(-3, 4, size=(K, N))
    C0 = rng.integers(-3, 4, size=(M, N))
    C, _ = ref(lib, A.astype(np.float32), B.astype(np.float32), C0.astype(np.float32),
               2.0, -1.0)
    want = 2 * (A @ B) - C0
    assert np.array_equal(C, want.astype(np.float64))
    # beta = 0.5 on integer C0 gives half-integers, still exact
    C, _ = ref(lib, A.astype(np.float32), B.astype(np.float32), C0.astype(np.float32),
               1.0, 0.5)
    assert np.array_equal(2.0 * C, (2 * (A @ B) + C0).astype(np.float64))


def _round_f32(x: Fraction) -> np.float32:
    """Exact rational -> nearest float32, ties to even (test helper)."""
    f = np.float32(float(x))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _near_midpoint(x: Fraction, tol: float) -> bool:
    f = np.float32(float(x))
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        for o in (np.nextafter(c, np.float32(-np.inf)), np.nextafter(c, np.float32(np.inf))):
            mid = (Fraction(float(c)) + Fraction(float(o))) / 2
            if abs(mid - x) <= Fraction(tol):
                return True
    return False


def test_brute_force_exact_rationals(lib):
    # Every shape with M, N, K in {0,1,2,3,5,8}, values U[-1,1), against exact
    # rational arithmetic on the same FP32 inputs.
    sizes = [0, 1, 2, 3, 5, 8]
    rng = np.random.default_rng(12)
    alpha, beta = np.float32(0.75), np.float32(-1.25)
    for M, N, K in itertools.product(sizes, sizes, sizes):
        A = draw(rng, (M, K), "uniform")
        B = draw(rng, (K, N), "uniform")
        C0 = draw(rng, (M, N), "uniform")
        C, babs = ref(lib, A, B, C0, float(alpha), float(beta), M=M, N=N, K=K)
        assert C.shape == (M, N)
        for i in range(M):
            for j in range(N):
                ps = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)]
                exact = Fraction(float(alpha)) * sum(ps, Fraction(0)) + \
                    Fraction(float(beta)) * Fraction(float(C0[i, j]))
                mag = abs(Fraction(float(alpha))) * sum((abs(p) for p in ps), Fraction(0)) + \
                    abs(Fraction(float(beta))) * abs(Fraction(float(C0[i, j])))
                tol = (K + 2) * U_D * float(mag) * 1.01
                assert abs(Fraction(C[i, j]) - exact) <= Fraction(tol), (M, N, K, i, j)
                assert abs(Fraction(babs[i, j]) - mag) <= Fraction(tol), (M, N, K, i, j)
                c32 = np.float32(C[i, j])
                if not _near_midpoint(exact, tol):
                    assert c32 == _round_f32(exact), (M, N, K, i, j)


def test_numpy_float64_crosscheck(lib):
    # Special case reducing to a library routine: a float64 matmul of the same
    # inputs is within 2*K*2^-53*Babs of the oracle (both are within K*u*Babs
    # of the exact result, in different summation orders).
    for (M, N, K), seed in [((67, 45, 300), 13), ((5, 300, 1024), 14), ((128, 1, 77), 15)]:
        A = rng_mat(seed, M, K)
        B = rng_mat(seed + 100, K, N, "normal")
        C, babs = ref(lib, A, B)
        L = A.astype(np.float64) @ B.astype(np.float64)
        assert np.all(np.abs(C - L) <= 2 * K * U_D * babs + 1e-300)


def test_linearity_in_alpha_beta(lib):
    A, B, C0 = rng_mat(16, 33, 65), rng_mat(17, 65, 21), rng_mat(18, 33, 21)
    C10, _ = ref(lib, A, B)
    for alpha, beta in [(2.0, -1.0), (0.5, 0.5), (-1.0, 2.0), (3.0, 0.25)]:
        C, _ = ref(lib, A, B, C0, alpha, beta)
        lin = alpha * C10 + beta * C0.astype(np.float64)
        # powers-of-two and small-integer scalars: one double rounding at most
        assert np.all(np.abs(C - lin) <= 4 * U_D * (np.abs(alpha * C10) + np.abs(beta * C0)))
    # integer inputs: exact
    Ai = rng_mat(19, 20, 30, "integer")
    Bi = rng_mat(20, 30, 10, "integer")
    Ci = rng_mat(21, 20, 10, "integer")
    C10, _ = ref(lib, Ai, Bi)
    for alpha, beta in [(2.0, -1.0), (0.5, 0.5), (-1.0, 2.0)]:
        C, _ = ref(lib, Ai, Bi, Ci, alpha, beta)
        assert np.array_equal(C, alpha * C10 + beta * Ci.astype(np.float64))


def test_quick_returns_and_nan_rules(lib):
    A, B, C0 = rng_mat(22, 6, 5), rng_mat(23, 5, 4), rng_mat(24, 6, 4)
    # M = 0 or N = 0: empty results
    C, _ = ref(lib, A[:0], B)
    assert C.shape == (0, 4)
    C, _ = ref(lib, A, B[:, :0])
    assert C.shape == (6, 0)
    # K = 0: C = beta*C0 (A and B not read)
    C, _ = ref(lib, A[:, :0], B[:0], C0, 1.5, -2.0)
    assert np.array_equal(C, -2.0 * C0.astype(np.float64))
    # alpha = 0: A and B are not read, even if they hold NaN
    An = np.full_like(A, np.nan)
    Bn = np.full_like(B, np.nan)
    C, babs = ref(lib, An, Bn, C0, 0.0, 0.5)
    assert np.array_equal(C, 0.5 * C0.astype(np.float64))
    assert np.array_equal(babs, 0.5 * np.abs(C0.astype(np.float64)))
    # beta = 0: C0 is not read, even if it holds NaN
    Cn = np.full_like(C0, np.nan)
    C, _ = ref(lib, A, B, Cn, 1.0, 0.0)
    assert np.all(np.isfinite(C))
    C2, _ = ref(lib, A, B)
    assert np.array_equal(C, C2)


def test_transpose_identity(lib):
    # (A B)^T = B^T A^T element by element with the same k order, so the two
    # evaluations agree bit for bit in double.
    A, B = rng_mat(25, 31, 47), rng_mat(26, 47, 19, "normal")
    C, babs = ref(lib, A, B)
    Ct, babst = ref(lib, np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(C, Ct.T) and np.array_equal(babs, babst.T)


def test_row_and_column_subsets_match_full(lib):
    A, B, C0 = rng_mat(27, 40, 33), rng_mat(28, 33, 50), rng_mat(29, 40, 50)
    C, babs = ref(lib, A, B, C0, 1.0, 0.5)
    rows = [0, 39, 17, 17, 5]
    cols = [49, 0, 20, 21]
    Cr, br = oracle.sgemm_ref_rows(A, B, C0, 1.0, 0.5, rows, lib=lib)
    Cc, bc = oracle.sgemm_ref_cols(A, B, C0, 1.0, 0.5, cols, lib=lib)
    assert np.array_equal(Cr, C[rows]) and np.array_equal(br, babs[rows])
    assert np.array_equal(Cc, C[:, cols]) and np.array_equal(bc, babs[:, cols])


def test_magnitude_sum_equals_value_for_nonnegative_inputs(lib):
    A = np.abs(rng_mat(30, 21, 63))
    B = np.abs(rng_mat(31, 63, 17))
    C0 = np.abs(rng_mat(32, 21, 17))
    C, babs = ref(lib, A, B, C0, 1.0, 1.0)
    assert np.array_equal(C, babs)


def test_strided_operands_match_packed(lib):
    M, N, K = 29, 31, 37
    Abuf = draw_matrix(33, M, K, "uniform", ld=K + 5)
    Bbuf = draw_matrix(34, K, N, "uniform", ld=N + 9)
    Cbuf = draw_matrix(35, M, N, "uniform", ld=N + 2)
    A, B, C0 = Abuf[:, :K], Bbuf[:, :N], Cbuf[:, :N]
    C, babs = ref(lib, A, B, C0, 1.0, 0.5)
    assert np.all(np.isfinite(C))
    Cp, bp = ref(lib, np.ascontiguousarray(A), np.ascontiguousarray(B),
                 np.ascontiguousarray(C0), 1.0, 0.5)
    assert np.array_equal(C, Cp) and np.array_equal(babs, bp)


def test_rejects_bad_arguments(lib):
    A, B = rng_mat(36, 4, 4), rng_mat(37, 4, 4)
    with pytest.raises(ValueError):
        ref(lib, A, B, M=-1)
    with pytest.raises(ValueError):
        oracle.sgemm_ref_rows(A, B, None, 1.0, 0.0, [4], lib=lib)
    with pytest.raises(ValueError):
        oracle.sgemm_ref_cols(A, B, None, 1.0, 0.0, [-1], lib=lib)


def test_views_whose_strides_numpy_does_not_canonicalise():
    # A transposed (n, 1) column is a (1, n) view with a row stride of one
    # float; numpy calls it C-contiguous as it stands. The oracle must still
    # read it as a row of n values (as C0, B or A), and a (1, 1) view with a
    # column stride of two floats as its one value.
    n = 939
    col = np.arange(n, dtype=np.float32).reshape(n, 1)
    row = col.T
    assert row.strides[0] < 4 * n
    a = np.full((4, 2), 3.0, np.float32)[:1, ::2]          # (1, 1), strides (8, 8)
    Cref, _ = oracle.sgemm_ref(a, row, row, 1.0, 0.5)
    assert np.array_equal(Cref[0], 3.0 * np.arange(n) + 0.5 * np.arange(n))
    Cref2, _ = oracle.sgemm_ref(row, col, None, 1.0, 0.0)   # 1 x n times n x 1: a dot product
    assert Cref2.shape == (1, 1) and Cref2[0, 0] == float(np.dot(np.arange(n, dtype=np.float64),
                                                                   np.arange(n, dtype=np.float64)))
