"""Host-side checks of the layout / transposition entry points (sgemm_f32_ex,
sgemm_f32_variant_ex, sgemm_f32_plan_ex): argument rules for every layout
and transposition, the column-major swap as the plan sees it, and which
kernels may run a transposed operand. No call here launches a kernel: the
argument errors and the unsupported-variant error are decided before any HIP
call, and the plan is host-only."""
import itertools

import pytest

import fp32_gemm_tuning_amd as sg

P = 1 << 20   # a fake, 16-byte aligned device address
ROW, COL = sg.ROW_MAJOR, sg.COL_MAJOR
NT, T = sg.NO_TRANS, sg.TRANS
TRANS_KERNELS = {"mfma_128x128", "mfma_256x256", "mfma_64x128", "mfma_64x128_kg4",
                 "mfma_64x96_kg4", "mfma_96x64_kg4", "mfma_128x128_kg4", "mfma_128x128_sk", "mfma_64x128_sk",
                 "mfma_256x256_sk", "mfma_64x64", "mfma_skinny", "mfma_direct"}


def min_lds(layout, ta, tb, M, N, K):
    """Smallest lda, ldb, ldc for each layout and transposition (CBLAS rules):
    the stored matrix's column count (row-major) or row count (column-major)."""
    a_rows, a_cols = (K, M) if ta else (M, K)
    b_rows, b_cols = (N, K) if tb else (K, N)
    if layout == ROW:
        return max(1, a_cols), max(1, b_cols), max(1, N)
    return max(1, a_rows), max(1, b_rows), max(1, M)


COMBOS = list(itertools.product((ROW, COL), (NT, T), (NT, T)))


@pytest.mark.parametrize("layout,ta,tb", COMBOS)
def test_leading_dimension_rules(layout, ta, tb):
    M, N, K = 5, 7, 3
    lda, ldb, ldc = min_lds(layout, ta, tb, M, N, K)
    ok = (layout, ta, tb, M, N, K, 1.0, P, lda, P, ldb, 0.0, P, ldc)
    assert sg.sgemm_f32_plan_ex(*ok, 256)[0] == 0
    for idx, code in ((8, -6), (10, -8), (13, -11)):
        bad = list(ok)
        bad[idx] -= 1
        assert sg.sgemm_f32_plan_ex(*bad, 256)[0] == code, (idx, bad)
        assert sg.sgemm_f32_ex(*bad, stream=0) == code
        assert sg.sgemm_f32_variant_ex(0, *bad, stream=0) == code


@pytest.mark.parametrize("args,code", [
    ((2, NT, NT), -13), ((-1, NT, NT), -13), ((ROW, 2, NT), -14), ((ROW, NT, -1), -15),
    ((COL, 7, 9), -14),
])
def test_flag_errors_come_first(args, code):
    # Flags precede M in the signature, so they are reported before a bad M.
    call = (*args, -1, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4)
    assert sg.sgemm_f32_ex(*call, stream=0) == code
    assert sg.sgemm_f32_variant_ex(7, *call, stream=0) == code
    assert sg.sgemm_f32_plan_ex(*call, 256)[0] == code
    assert "neither" in sg.sgemm_f32_strerror(code)


def test_ex_matches_sgemm_f32_on_the_plain_case():
    for (M, N, K) in ((4096, 4096, 4096), (1000, 1531, 777), (8, 4096, 4096), (256, 256, 256)):
        a = (M, N, K, 1.0, P, K, P, N, 0.0, P, N)
        assert sg.sgemm_f32_plan_ex(ROW, NT, NT, *a, 256) == sg.sgemm_f32_plan(*a, 256)
    # the same argument errors
    bad = (4, 4, 8, 1.0, P, 7, P, 4, 0.0, P, 4)
    assert sg.sgemm_f32_ex(ROW, NT, NT, *bad, stream=0) == sg.sgemm_f32(*bad, stream=0) == -6


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (1000, 1531, 777), (8, 4096, 4096),
                                   (4096, 8, 4096), (256, 256, 256), (2048, 2048, 2048)])
def test_column_major_plain_call_is_the_swapped_row_major_call(M, N, K):
    # C (M x N, col-major) = A B is C^T = B^T A^T row-major: an N x M product
    # with the operands swapped and nothing transposed, so every kernel,
    # including the skinny one (for small N), is available.
    # The exception: few rows and more columns, which the skinny kernel takes
    # unswapped (after the swap it would be a product with few columns).
    rc, v = sg.sgemm_f32_plan_ex(COL, NT, NT, M, N, K, 1.0, P, M, P, K, 0.0, P, M, 256)
    assert rc == 0
    if M <= 32 < N:
        assert sg.sgemm_f32_variant_name(v) == "mfma_skinny"
    else:
        assert (rc, v) == sg.sgemm_f32_plan(N, M, K, 1.0, P, K, P, M, 0.0, P, M, 256)


@pytest.mark.parametrize("layout,ta,tb", [c for c in COMBOS if c not in ((ROW, NT, NT), (COL, NT, NT))])
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (1000, 1531, 777), (8, 4096, 4096),
                                   (4096, 8, 4096), (256, 256, 256), (1, 1, 1), (2048, 2048, 2048)])
def test_transposed_calls_plan_a_kernel_that_reads_them(layout, ta, tb, M, N, K):
    lda, ldb, ldc = min_lds(layout, ta, tb, M, N, K)
    rc, v = sg.sgemm_f32_plan_ex(layout, ta, tb, M, N, K, 1.0, P, lda, P, ldb, 0.0, P, ldc, 256)
    assert rc == 0
    assert sg.sgemm_f32_variant_name(v) in TRANS_KERNELS
    assert sg.sgemm_f32_variant_trans_ok(v) == 1


def test_transposed_plan_follows_the_model():
    # The large square case takes the 256x256 kernel whether or not an
    # operand is transposed; the odd case one of the K-group kernels.
    for ta, tb in ((T, NT), (NT, T), (T, T)):
        lda, ldb, ldc = min_lds(ROW, ta, tb, 4096, 4096, 4096)
        _, v = sg.sgemm_f32_plan_ex(ROW, ta, tb, 4096, 4096, 4096, 1.0, P, lda, P, ldb, 0.0, P,
                                    ldc, 256)
        assert sg.sgemm_f32_variant_name(v) == "mfma_256x256"
        lda, ldb, ldc = min_lds(ROW, ta, tb, 1000, 1531, 777)
        _, v = sg.sgemm_f32_plan_ex(ROW, ta, tb, 1000, 1531, 777, 1.0, P, lda, P, ldb, 0.0, P,
                                    ldc, 256)
        assert sg.sgemm_f32_variant_name(v) == sg.sgemm_f32_variant_name(
            sg.sgemm_f32_plan(1000, 1531, 777, 1.0, P, 777, P, 1531, 0.0, P, 1531, 256)[1])


@pytest.mark.parametrize("layout,ta,tb", [c for c in COMBOS if c not in ((ROW, NT, NT), (COL, NT, NT))])
def test_transposed_few_rows_and_tiny_calls_take_the_small_kernels(layout, ta, tb):
    # M <= 32 rows (N <= 32 columns for column-major: rows after the swap)
    # take the skinny kernel and tiny products the direct one, transposed or not.
    for (M, N, K), want in (((16, 8192, 8192), "mfma_skinny"), ((256, 256, 256), "mfma_direct")):
        if layout == COL:
            M, N = N, M
        lda, ldb, ldc = min_lds(layout, ta, tb, M, N, K)
        rc, v = sg.sgemm_f32_plan_ex(layout, ta, tb, M, N, K, 1.0, P, lda, P, ldb, 0.0, P, ldc, 256)
        assert rc == 0 and sg.sgemm_f32_variant_name(v) == want, (M, N, K)


@pytest.mark.parametrize("ta,tb", [(NT, NT), (T, NT), (NT, T), (T, T)])
def test_column_major_few_rows_take_the_skinny_kernel(ta, tb):
    # 16 rows, 8192 columns, column-major: the skinny kernel, unswapped; with
    # few columns as well the swapped call is itself a few-row product.
    for (M, N, K) in ((16, 8192, 8192), (32, 33, 100), (7, 4096, 1029), (16, 16, 4096)):
        lda, ldb, ldc = min_lds(COL, ta, tb, M, N, K)
        rc, v = sg.sgemm_f32_plan_ex(COL, ta, tb, M, N, K, 1.0, P, lda, P, ldb, 0.0, P, ldc, 256)
        assert rc == 0 and sg.sgemm_f32_variant_name(v) == "mfma_skinny", (M, N, K)
    # A leading dimension too large for the skinny kernel's 32-bit buffer
    # offsets (the 31 rows a 32-deep block of the stored A^T spans past its
    # first cover more than 2^31 bytes): the call keeps the swapped plan
    # instead.
    if (ta, tb) == (NT, NT):
        rc, v = sg.sgemm_f32_plan_ex(COL, NT, NT, 16, 8192, 8192, 1.0, P, 1 << 25, P, 8192, 0.0, P,
                                     16, 256)
        assert rc == 0 and sg.sgemm_f32_variant_name(v) != "mfma_skinny"
    # Row-major with few columns is the same transposed problem.
    for (M, N, K) in ((8192, 16, 8192), (4096, 8, 4096), (33, 32, 100)):
        lda, ldb, ldc = min_lds(ROW, ta, tb, M, N, K)
        rc, v = sg.sgemm_f32_plan_ex(ROW, ta, tb, M, N, K, 1.0, P, lda, P, ldb, 0.0, P, ldc, 256)
        assert rc == 0 and sg.sgemm_f32_variant_name(v) == "mfma_skinny", (M, N, K)
    # 33 rows are not few
    lda, ldb, ldc = min_lds(COL, ta, tb, 33, 8192, 8192)
    rc, v = sg.sgemm_f32_plan_ex(COL, ta, tb, 33, 8192, 8192, 1.0, P, lda, P, ldb, 0.0, P, ldc, 256)
    assert rc == 0 and sg.sgemm_f32_variant_name(v) != "mfma_skinny"


def test_trans_ok_flags():
    for i, name in enumerate(sg.VARIANTS):
        assert sg.sgemm_f32_variant_trans_ok(i) == (1 if name in TRANS_KERNELS else 0), name
    assert sg.sgemm_f32_variant_trans_ok(-1) == sg.ERR_VARIANT
    assert sg.sgemm_f32_variant_trans_ok(len(sg.VARIANTS)) == sg.ERR_VARIANT


@pytest.mark.parametrize("name", [n for n in sg.VARIANTS if n not in TRANS_KERNELS])
def test_kernels_without_transposed_reads_refuse(name):
    v = sg.sgemm_f32_variant_by_name(name)
    # row-major, A transposed: refused before any launch
    assert sg.sgemm_f32_variant_ex(v, ROW, T, NT, 64, 64, 64, 1.0, P, 64, P, 64, 0.0, P, 64,
                                   stream=0) == sg.ERR_UNSUPPORTED
    # column-major, B transposed: after the swap A is transposed; refused
    assert sg.sgemm_f32_variant_ex(v, COL, NT, T, 64, 64, 64, 1.0, P, 64, P, 64, 0.0, P, 64,
                                   stream=0) == sg.ERR_UNSUPPORTED


def test_transposed_plan_with_a_model_that_has_no_candidate():
    # Every model kernel reads transposed operands; a call that the model's
    # only entry cannot take (here mfma_256x256 with 4-byte fills, an instance
    # that spills) falls back to mfma_128x128, transposed or not.
    try:
        assert sg.sgemm_f32_set_model([{"variant": "mfma_256x256", "overhead_us": 1.0,
                                        "eff": [0.5, 0.5, 0.5, 0.5]}]) == 0
        rc, v = sg.sgemm_f32_plan_ex(ROW, T, NT, 512, 512, 513, 1.0, P, 513, P, 512, 0.0, P, 512,
                                     256)
        assert rc == 0 and sg.sgemm_f32_variant_name(v) == "mfma_128x128"
        rc, v = sg.sgemm_f32_plan_ex(ROW, T, NT, 512, 512, 512, 1.0, P, 512, P, 512, 0.0, P, 512,
                                     256)
        assert rc == 0 and sg.sgemm_f32_variant_name(v) == "mfma_256x256"
    finally:
        assert sg.sgemm_f32_set_model([]) == 0


def test_quick_returns_and_null_operands():
    # M == 0: nothing read or written, for every layout and transposition
    for layout, ta, tb in COMBOS:
        assert sg.sgemm_f32_ex(layout, ta, tb, 0, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, stream=0) == 0
        rc, v = sg.sgemm_f32_plan_ex(layout, ta, tb, 4, 4, 4, 0.0, 0, 4, 0, 4, 1.0, P, 4, 256)
        assert (rc, v) == (0, -1)


def test_plan_ex_null_output():
    assert sg.lib().sgemm_f32_plan_ex(ROW, T, NT, 4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4, 256,
                                      None) == -12
