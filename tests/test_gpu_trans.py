"""GPU parity of the layout / transposition entry points against the FP64
oracle. The operands are drawn as the matrices the caller stores (row- or
column-major, transposed or not, with NaN-filled padding past each leading
dimension's used extent); the oracle gets op(A), op(B) and C0 as plain
row-major copies made here on the host (materialising a transpose is a copy,
not arithmetic). Bars as for the untransposed calls: integer-valued inputs bit
for bit, random ones within 4*K*2^-24*Babs elementwise and a relative
Frobenius error of 1e-5."""
import itertools

import numpy as np
import pytest

import oracle
from datagen import WORKLOADS, draw_matrix
from oracle.compare import check_bound, check_exact

torch = pytest.importorskip("torch")
import fp32_gemm_tuning_amd as sg  # noqa: E402

pytestmark = pytest.mark.gpu

ROW, COL = sg.ROW_MAJOR, sg.COL_MAJOR
NT, T = sg.NO_TRANS, sg.TRANS
COMBOS = list(itertools.product((ROW, COL), (NT, T), (NT, T)))
TRANS_KERNELS = ["mfma_128x128", "mfma_256x256", "mfma_64x128", "mfma_64x128_kg4",
                 "mfma_64x96_kg4", "mfma_96x64_kg4", "mfma_128x128_kg4", "mfma_128x128_sk", "mfma_64x128_sk",
                 "mfma_256x256_sk", "mfma_64x64", "mfma_skinny", "mfma_direct"]


def combo_id(c):
    return ("row" if c[0] == ROW else "col") + "-" + ("T" if c[1] else "N") + ("T" if c[2] else "N")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    return torch.device("cuda:0")


class Stored:
    """A rows x cols matrix as the caller stores it in `layout` order: `buf`
    is the row-major buffer (rows x ld for row-major, cols x ld for
    column-major), `ld` its leading dimension, `logical` the rows x cols
    matrix as a row-major copy."""

    def __init__(self, layout, rows, cols, dist, seed, pad, fill=None):
        if layout == ROW:
            outer, inner = rows, cols
        else:
            outer, inner = cols, rows
        self.ld = inner + pad
        if fill is None:
            self.buf = draw_matrix(seed, outer, inner, dist, ld=self.ld)
        else:
            self.buf = np.full((outer, self.ld), fill, np.float32)
        used = self.buf[:, :inner]
        self.logical = np.ascontiguousarray(used if layout == ROW else used.T)
        self.layout, self.inner = layout, inner

    def read_logical(self, buf):
        used = buf[:, :self.inner]
        return np.ascontiguousarray(used if self.layout == ROW else used.T)


def make_case(layout, ta, tb, M, N, K, dist, seed, beta, pads):
    A = Stored(layout, K if ta else M, M if ta else K, dist, seed, pads[0])
    B = Stored(layout, N if tb else K, K if tb else N, dist, seed + 1, pads[1])
    if beta != 0.0:
        C = Stored(layout, M, N, dist, seed + 2, pads[2])
    else:
        C = Stored(layout, M, N, dist, seed + 2, pads[2], fill=np.nan)
    opA = np.ascontiguousarray(A.logical.T) if ta else A.logical
    opB = np.ascontiguousarray(B.logical.T) if tb else B.logical
    return A, B, C, opA, opB


def to_dev(buf, dev, offset=0):
    flat = torch.empty(buf.size + offset, dtype=torch.float32, device=dev)
    flat[offset:] = torch.from_numpy(np.ascontiguousarray(buf).ravel()).to(dev)
    return flat, flat.data_ptr() + 4 * offset


def run_ex(variant, layout, ta, tb, M, N, K, alpha, beta, A, B, C, dev, offsets=(0, 0, 0),
           tag=""):
    fa, pa = to_dev(A.buf, dev, offsets[0])
    fb, pb = to_dev(B.buf, dev, offsets[1])
    fc, pc = to_dev(C.buf, dev, offsets[2])
    name = "auto" if variant is None else variant
    # stream-K kernels get the workspace they ask for
    vid = -1 if variant is None else sg.sgemm_f32_variant_by_name(variant)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    rc, wsb = sg.sgemm_f32_ws_size(vid, layout, ta, tb, M, N, K, cus)
    assert rc == 0
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    print(f"[gpu] {tag} ex variant={name} layout={layout} ta={ta} tb={tb} M={M} N={N} K={K} "
          f"ld=({A.ld},{B.ld},{C.ld}) off={offsets} ws={wsb}", flush=True)
    s = torch.cuda.current_stream()
    if variant is None:
        rc = sg.sgemm_f32_ex(layout, ta, tb, M, N, K, alpha, pa, A.ld, pb, B.ld, beta, pc, C.ld,
                             s.cuda_stream)
    else:
        rc = sg.sgemm_f32_variant_ws(vid, layout, ta, tb, M, N, K, alpha, pa, A.ld, pb, B.ld,
                                     beta, pc, C.ld, ws, wsb, s.cuda_stream)
    torch.cuda.synchronize()
    out = fc[offsets[2]:].cpu().numpy().reshape(C.buf.shape)
    del fa, fb, fc, ws
    return rc, out


def check(out, C, opA, opB, M, N, K, alpha, beta, exact):
    Cref, babs = oracle.sgemm_ref(opA, opB, C.logical if beta != 0.0 else None, alpha, beta,
                                  M=M, N=N, K=K)
    got = C.read_logical(out)
    rep = check_exact(got, Cref) if exact else check_bound(got, Cref, babs, K)
    # the padding of C is never written
    assert np.array_equal(out[:, C.inner:], C.buf[:, C.inner:], equal_nan=True)
    return rep


# (M, N, K, alpha, beta, dist, pads, offsets): 16-byte fills where the
# contiguous extents and leading dimensions allow them, 4-byte fills on odd
# sizes and misaligned bases, full tiles of every kernel, one K slice.
SMALL = [
    (256, 256, 256, 1.0, 0.0, "integer", (0, 0, 0), (0, 0, 0)),
    (300, 260, 100, 1.5, -0.5, "uniform", (4, 8, 7), (0, 0, 0)),
    (129, 131, 67, 1.0, 0.5, "integer", (3, 5, 1), (0, 0, 0)),
    (260, 272, 16, 1.0, 0.0, "integer", (0, 0, 0), (0, 0, 0)),
    (200, 136, 64, 1.0, 0.25, "integer", (0, 0, 0), (1, 3, 2)),
    (513, 385, 250, 1.0, 0.0, "normal", (0, 0, 0), (0, 0, 0)),
]


@pytest.mark.parametrize("combo", COMBOS, ids=combo_id)
@pytest.mark.parametrize("variant", TRANS_KERNELS)
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:3])) + f"-{c[5]}")
def test_transposed_small(dev, combo, variant, case):
    layout, ta, tb = combo
    M, N, K, alpha, beta, dist, pads, offsets = case
    A, B, C, opA, opB = make_case(layout, ta, tb, M, N, K, dist, 500 + M + N + K, beta, pads)
    rc, out = run_ex(variant, layout, ta, tb, M, N, K, alpha, beta, A, B, C, dev, offsets,
                     tag="trans-small")
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    rep = check(out, C, opA, opB, M, N, K, alpha, beta, exact=(dist == "integer"))
    assert rep.ok, f"{variant} {combo_id(combo)} {case}: {rep}"


# Few rows and long K for the kernels that load their k-runs straight from
# memory: K spread over all 16 waves of mfma_skinny with a ragged last run,
# 16-byte k-runs where the stored rows allow them, 4-byte ones on odd pitches
# and misaligned bases.
SMALL_M = [
    (16, 520, 4100, 1.0, 0.0, "uniform", (0, 0, 0), (0, 0, 0)),
    (32, 64, 4096, 1.0, 0.5, "integer", (0, 0, 0), (0, 0, 0)),
    (7, 333, 1029, 2.0, -1.0, "integer", (1, 3, 2), (1, 0, 3)),
    (20, 96, 52, 1.0, 0.0, "integer", (4, 0, 0), (0, 2, 0)),
]


@pytest.mark.parametrize("combo", COMBOS, ids=combo_id)
@pytest.mark.parametrize("variant", ["mfma_skinny", "mfma_direct"])
@pytest.mark.parametrize("case", SMALL_M, ids=lambda c: "x".join(map(str, c[:3])) + f"-{c[5]}")
def test_transposed_few_rows(dev, combo, variant, case):
    layout, ta, tb = combo
    M, N, K, alpha, beta, dist, pads, offsets = case
    if layout == COL:
        M, N = N, M   # few columns: few rows after the column-major swap
    A, B, C, opA, opB = make_case(layout, ta, tb, M, N, K, dist, 700 + M + N + K, beta, pads)
    rc, out = run_ex(variant, layout, ta, tb, M, N, K, alpha, beta, A, B, C, dev, offsets,
                     tag="trans-few-rows")
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    rep = check(out, C, opA, opB, M, N, K, alpha, beta, exact=(dist == "integer"))
    assert rep.ok, f"{variant} {combo_id(combo)} {case}: {rep}"


@pytest.mark.parametrize("layout", [COL, ROW], ids=["col", "row"])
@pytest.mark.parametrize("ta,tb", [(NT, NT), (T, NT), (NT, T), (T, T)], ids=["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("case", SMALL_M, ids=lambda c: "x".join(map(str, c[:3])) + f"-{c[5]}")
def test_few_rows_or_columns_auto(dev, layout, ta, tb, case):
    # Few rows in column-major storage, or few columns in row-major storage:
    # the automatic choice runs the skinny kernel on the transposed problem
    # (few rows), reading both operands as transposes and writing C^T
    # column-major.
    M, N, K, alpha, beta, dist, pads, offsets = case
    if layout == ROW:
        M, N = N, M
    A, B, C, opA, opB = make_case(layout, ta, tb, M, N, K, dist, 800 + M + N + K, beta, pads)
    rc, v = sg.sgemm_f32_plan_ex(layout, ta, tb, M, N, K, alpha, 1 << 20, A.ld, 1 << 20, B.ld, beta,
                                 1 << 20, C.ld, 256)
    assert rc == 0 and sg.sgemm_f32_variant_name(v) == "mfma_skinny"
    rc, out = run_ex(None, layout, ta, tb, M, N, K, alpha, beta, A, B, C, dev, offsets,
                     tag="few-rows-or-columns")
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    rep = check(out, C, opA, opB, M, N, K, alpha, beta, exact=(dist == "integer"))
    assert rep.ok, f"{combo_id((layout, ta, tb))} {case}: {rep}"


@pytest.mark.parametrize("variant", sg.VARIANTS)
def test_column_major_plain_runs_every_variant(dev, variant):
    # Column-major with nothing transposed is the swapped row-major product
    # (here 200 x 132 x 68, ragged for every tile): every kernel runs it.
    # The sizes keep the rows 16-byte aligned after the swap, which
    # vec4_transa needs.
    M, N, K = 132, 200, 68
    A, B, C, opA, opB = make_case(COL, NT, NT, M, N, K, "integer", 77, 0.5, (0, 0, 0))
    rc, out = run_ex(variant, COL, NT, NT, M, N, K, 1.0, 0.5, A, B, C, dev, tag="col-plain")
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    rep = check(out, C, opA, opB, M, N, K, 1.0, 0.5, exact=True)
    assert rep.ok, f"{variant}: {rep}"


@pytest.mark.parametrize("combo", COMBOS, ids=combo_id)
@pytest.mark.parametrize("shape", [(1000, 1531, 777), (8, 4096, 1024), (4096, 8, 1024),
                                   (1, 1, 1), (33, 70, 1000)])
def test_transposed_auto(dev, combo, shape):
    layout, ta, tb = combo
    M, N, K = shape
    A, B, C, opA, opB = make_case(layout, ta, tb, M, N, K, "uniform", 900 + M, 0.0, (0, 0, 0))
    rc, out = run_ex(None, layout, ta, tb, M, N, K, 1.0, 0.0, A, B, C, dev, tag="trans-auto")
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    rep = check(out, C, opA, opB, M, N, K, 1.0, 0.0, exact=False)
    assert rep.ok, f"{combo_id(combo)} {shape}: {rep}"


@pytest.mark.parametrize("combo", [(ROW, T, NT), (ROW, NT, T), (ROW, T, T), (COL, NT, NT)],
                         ids=combo_id)
def test_transposed_headline_size(dev, combo):
    # 4096^3 through the automatic choice (the 256x256 kernel's full-tile
    # instance), every element checked.
    layout, ta, tb = combo
    w = WORKLOADS["S4096"]
    M, N, K = w.M, w.N, w.K
    A, B, C, opA, opB = make_case(layout, ta, tb, M, N, K, "uniform", 4096, 0.0, (0, 0, 0))
    rc, out = run_ex(None, layout, ta, tb, M, N, K, 1.0, 0.0, A, B, C, dev, tag="trans-S4096")
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    rep = check(out, C, opA, opB, M, N, K, 1.0, 0.0, exact=False)
    print(f"[gpu] S4096 {combo_id(combo)}: {rep}", flush=True)
    assert rep.n == M * N
    assert rep.ok, f"{combo_id(combo)}: {rep}"


@pytest.mark.parametrize("combo", [(COL, NT, NT), (COL, T, T), (ROW, T, NT), (ROW, NT, T)],
                         ids=combo_id)
def test_few_rows_full_size(dev, combo):
    # 16 x 8192 x 8192 (the near-GEMV workload) through the automatic choice:
    # column-major runs the skinny kernel unswapped, row-major with a
    # transposed operand reads it in place; every element checked.
    layout, ta, tb = combo
    w = WORKLOADS["R_skinny"]
    M, N, K = w.M, w.N, w.K
    A, B, C, opA, opB = make_case(layout, ta, tb, M, N, K, "uniform", 1600, 0.0, (0, 0, 0))
    rc, out = run_ex(None, layout, ta, tb, M, N, K, 1.0, 0.0, A, B, C, dev, tag="few-rows-R_skinny")
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    rep = check(out, C, opA, opB, M, N, K, 1.0, 0.0, exact=False)
    print(f"[gpu] R_skinny {combo_id(combo)}: {rep}", flush=True)
    assert rep.n == M * N
    assert rep.ok, f"{combo_id(combo)}: {rep}"


@pytest.mark.parametrize("ta,tb", [(NT, NT), (T, T)], ids=["NN", "TT"])
def test_few_columns_full_size(dev, ta, tb):
    # 8192 x 16 x 8192 row-major (the near-GEMV workload transposed): the
    # skinny kernel on C^T = B^T A^T; every element checked.
    w = WORKLOADS["R_skinny"]
    M, N, K = w.N, w.M, w.K
    A, B, C, opA, opB = make_case(ROW, ta, tb, M, N, K, "uniform", 1700, 0.0, (0, 0, 0))
    rc, out = run_ex(None, ROW, ta, tb, M, N, K, 1.0, 0.0, A, B, C, dev, tag="few-columns-full")
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    rep = check(out, C, opA, opB, M, N, K, 1.0, 0.0, exact=False)
    print(f"[gpu] R_skinny transposed row {ta}{tb}: {rep}", flush=True)
    assert rep.n == M * N
    assert rep.ok, rep


def test_gemm_helper_takes_transposed_views(dev):
    M, N, K = 300, 200, 100
    g = np.random.default_rng(5)
    At = g.integers(-3, 4, (K, M)).astype(np.float32)     # stores A^T
    Bt = g.integers(-3, 4, (N, K)).astype(np.float32)     # stores B^T
    C0 = g.integers(-3, 4, (M, N)).astype(np.float32)
    A_dev = torch.from_numpy(At).to(dev).t()               # M x K view, column-major
    B_dev = torch.from_numpy(Bt).to(dev).t()               # K x N view, column-major
    for c_col in (False, True):
        if c_col:
            C_dev = torch.from_numpy(np.ascontiguousarray(C0.T)).to(dev).t()   # column-major C
        else:
            C_dev = torch.from_numpy(C0.copy()).to(dev)
        print(f"[gpu] gemm helper, column-major C={c_col}", flush=True)
        sg.gemm(A_dev, B_dev, C_dev, alpha=2.0, beta=-1.0)
        torch.cuda.synchronize()
        Cref, _ = oracle.sgemm_ref(np.ascontiguousarray(At.T), np.ascontiguousarray(Bt.T), C0,
                                   2.0, -1.0)
        rep = check_exact(np.ascontiguousarray(C_dev.cpu().numpy()), Cref)
        assert rep.ok, rep


# Seeded random calls through the automatic choice, without a workspace
# (sgemm_f32_ex) and with one (sgemm_f32_ws): sides log-uniform in [1, 1200]
# (eight in [1200, 3000]), every storage order and transposition, padded
# leading dimensions, misaligned bases, alpha and beta from small sets;
# integer inputs (bit for bit) and uniform ones (the error bound). The
# dispatch takes every kernel family on some of them, each with its edge and
# fill paths.
def _random_cases(n, n_large, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n + n_large):
        hi = 1200 if i < n else 3000
        lo = 1 if i < n else 1200
        M, N, K = (int(round(np.exp(rng.uniform(np.log(lo), np.log(hi))))) for _ in range(3))
        layout, ta, tb = COMBOS[int(rng.integers(len(COMBOS)))]
        alpha = float(rng.choice([1.0, -1.0, 2.0, 0.5]))
        beta = float(rng.choice([0.0, 0.0, 1.0, 0.5, -2.0]))
        dist = "integer" if i % 2 == 0 else "uniform"
        pads = tuple(int(x) for x in rng.choice([0, 0, 1, 3, 4, 7], size=3))
        offsets = tuple(int(x) for x in rng.choice([0, 0, 0, 1, 2, 3], size=3))
        cases.append((M, N, K, alpha, beta, dist, pads, offsets, layout, ta, tb, bool(i % 3 == 0)))
    return cases


RANDOM = _random_cases(72, 8, 2026)


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: "x".join(map(str, c[:3])) + "-" +
                         combo_id(c[8:11]) + ("-ws" if c[11] else ""))
def test_random_calls_auto(dev, case):
    M, N, K, alpha, beta, dist, pads, offsets, layout, ta, tb, use_ws = case
    A, B, C, opA, opB = make_case(layout, ta, tb, M, N, K, dist, 900 + M + N + K, beta, pads)
    if not use_ws:
        rc, out = run_ex(None, layout, ta, tb, M, N, K, alpha, beta, A, B, C, dev, offsets,
                         tag="random")
    else:
        fa, pa = to_dev(A.buf, dev, offsets[0])
        fb, pb = to_dev(B.buf, dev, offsets[1])
        fc, pc = to_dev(C.buf, dev, offsets[2])
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        rc, wsb = sg.sgemm_f32_ws_size(-1, layout, ta, tb, M, N, K, cus)
        assert rc == 0
        ws = torch.full((max(wsb, 16),), 0xFF, dtype=torch.uint8, device=dev)
        print(f"[gpu] random ws layout={layout} ta={ta} tb={tb} M={M} N={N} K={K} "
              f"ld=({A.ld},{B.ld},{C.ld}) off={offsets} ws={wsb}", flush=True)
        rc = sg.sgemm_f32_ws(layout, ta, tb, M, N, K, alpha, pa, A.ld, pb, B.ld, beta, pc, C.ld,
                             ws, wsb, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        out = fc[offsets[2]:].cpu().numpy().reshape(C.buf.shape)
        del fa, fb, fc, ws
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    rep = check(out, C, opA, opB, M, N, K, alpha, beta, exact=(dist == "integer"))
    assert rep.ok, f"{case}: {rep}"
