"""GPU parity of the stream-K kernels (sgemm_f32_ws) against the FP64 oracle.

Each shape is chosen for the split it makes on the device (checked against
the tuner's copy of the split before launching): a single tile cut into three
pieces, runs of slices that cross tile boundaries, ragged edges with 4-byte
fills, whole tiles next to split ones, and one-slice tiles that are never
split. The workspace is filled with 0xFF bytes (NaN partials) before every
call, so a partial that is read before it is written shows up in the result.
Integer inputs must match bit for bit (their partial sums are exact in any
order); random ones meet the elementwise bound. Repeated calls must give
identical bits."""
import numpy as np
import pytest

import oracle
from datagen import draw_matrix
from oracle.compare import check_bound, check_exact

torch = pytest.importorskip("torch")
import fp32_gemm_tuning_amd as sg  # noqa: E402
from fp32_gemm_tuning_amd import tune  # noqa: E402

pytestmark = pytest.mark.gpu

SK = ["mfma_128x128_sk", "mfma_64x128_sk", "mfma_256x256_sk"]
ROW = sg.ROW_MAJOR


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def cus(dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


def to_dev(buf, dev):
    return torch.from_numpy(np.ascontiguousarray(buf)).to(dev)


def call_sk(variant, M, N, K, alpha, beta, A, B, C0, dev, cus, ta=0, tb=0, ws_extra=0,
            tag=""):
    """One sgemm_f32_variant_ws call (variant None: sgemm_f32_ws) on a
    poisoned workspace; returns (rc, C as numpy, workspace bytes)."""
    vid = -1 if variant is None else sg.sgemm_f32_variant_by_name(variant)
    rc, wsb = sg.sgemm_f32_ws_size(vid, ROW, ta, tb, M, N, K, cus)
    assert rc == 0
    wsb += ws_extra
    ws = torch.full((max(16, wsb),), 0xFF, dtype=torch.uint8, device=dev)
    dA, dB, dC = to_dev(A, dev), to_dev(B, dev), to_dev(C0, dev)
    print(f"[gpu] {tag} sk variant={variant or 'auto'} M={M} N={N} K={K} ta={ta} tb={tb} "
          f"ws={wsb}", flush=True)
    s = torch.cuda.current_stream()
    args = (ROW, ta, tb, M, N, K, alpha, dA, A.shape[1], dB, B.shape[1], beta, dC, C0.shape[1],
            ws, wsb, s.cuda_stream)
    rc = sg.sgemm_f32_ws(*args) if variant is None else sg.sgemm_f32_variant_ws(vid, *args)
    torch.cuda.synchronize()
    return rc, dC.cpu().numpy(), wsb


def operands(M, N, K, dist, seed, beta, ta=0, tb=0):
    A = draw_matrix(seed, K if ta else M, M if ta else K, dist)
    B = draw_matrix(seed + 1, N if tb else K, K if tb else N, dist)
    C0 = draw_matrix(seed + 2, M, N, dist) if beta != 0.0 else np.full((M, N), np.nan, np.float32)
    opA = np.ascontiguousarray(A.T) if ta else A
    opB = np.ascontiguousarray(B.T) if tb else B
    return A, B, C0, opA, opB


def split_of(variant, M, N, K, cus):
    bm, bn = tune.TILE[variant]
    tiles = -(-M // bm) * -(-N // bn)
    return tune.sk_split(tiles, -(-K // tune.SK_BK[variant]), cus)


# (M, N, K, alpha, beta, dist): see the module docstring for what each splits.
CASES = [
    (128, 128, 48, 1.0, 0.0, "integer"),      # one 128-tile, 3 slices -> 3 one-slice pieces
    (640, 128, 112, 1.0, 0.5, "integer"),     # 5 tiles x 7 slices, runs of 2 cross tiles
    (300, 260, 100, 1.5, -0.5, "uniform"),    # ragged everywhere
    (129, 131, 67, 1.0, 0.25, "integer"),     # 4-byte fills (odd sizes)
    (2176, 2176, 256, 1.0, 0.0, "integer"),   # 289 / 578 tiles: whole tiles + split ones
    (2176, 2176, 250, 1.0, 0.5, "uniform"),
    (700, 600, 16, 1.0, 0.0, "integer"),      # one slice per tile: never split
    (1000, 1531, 777, 1.0, 0.0, "uniform"),
    # tile grid and K slices exact for all three tiles (the unmasked instance),
    # still split into pieces that cross tiles
    (512, 512, 64, 1.0, 0.0, "integer"),
    (768, 512, 96, 1.0, 0.5, "uniform"),
]


@pytest.mark.parametrize("variant", SK)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"-{c[5]}")
def test_stream_k_parity(dev, cus, variant, case):
    M, N, K, alpha, beta, dist = case
    A, B, C0, opA, opB = operands(M, N, K, dist, 40 + M + K, beta)
    rc, C, wsb = call_sk(variant, M, N, K, alpha, beta, A, B, C0, dev, cus, tag="sk")
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    sp = split_of(variant, M, N, K, cus)
    assert (wsb > 0) == (sp is not None)
    Cref, babs = oracle.sgemm_ref(opA, opB, C0 if beta != 0.0 else None, alpha, beta)
    rep = check_exact(C, Cref) if dist == "integer" else check_bound(C, Cref, babs, K)
    print(f"[gpu] {variant} {case[:3]} split={sp}: {rep}", flush=True)
    assert rep.ok, f"{variant} {case}: {rep}"


@pytest.mark.parametrize("variant", SK)
@pytest.mark.parametrize("ta,tb", [(1, 0), (0, 1), (1, 1)])
def test_stream_k_transposed(dev, cus, variant, ta, tb):
    M, N, K = 640, 384, 200
    A, B, C0, opA, opB = operands(M, N, K, "integer", 77, 1.0, ta, tb)
    rc, C, wsb = call_sk(variant, M, N, K, 1.0, 1.0, A, B, C0, dev, cus, ta, tb, tag="sk-trans")
    assert rc == 0 and wsb > 0, sg.sgemm_f32_strerror(rc)
    Cref, _ = oracle.sgemm_ref(opA, opB, C0, 1.0, 1.0)
    rep = check_exact(C, Cref)
    assert rep.ok, f"{variant} ta={ta} tb={tb}: {rep}"


@pytest.mark.parametrize("variant", SK)
def test_stream_k_is_deterministic(dev, cus, variant):
    M, N, K = 2176, 2176, 250
    A, B, C0, _, _ = operands(M, N, K, "uniform", 5, 0.0)
    rc1, C1, _ = call_sk(variant, M, N, K, 1.0, 0.0, A, B, C0, dev, cus, tag="sk-det-1")
    rc2, C2, _ = call_sk(variant, M, N, K, 1.0, 0.0, A, B, C0, dev, cus, ws_extra=4096,
                         tag="sk-det-2")
    assert rc1 == rc2 == 0
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


def test_stream_k_needs_its_workspace(dev, cus):
    M, N, K = 640, 128, 112
    v = sg.sgemm_f32_variant_by_name("mfma_128x128_sk")
    _, need = sg.sgemm_f32_ws_size(v, ROW, 0, 0, M, N, K, cus)
    assert need > 0
    A = torch.zeros(M, K, device=dev)
    B = torch.zeros(K, N, device=dev)
    C = torch.zeros(M, N, device=dev)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    print("[gpu] sk workspace too small", flush=True)
    assert sg.sgemm_f32_variant_ws(v, ROW, 0, 0, M, N, K, 1.0, A, K, B, N, 0.0, C, N, ws,
                                   need - 1) == sg.ERR_WORKSPACE
    assert sg.sgemm_f32_variant(v, M, N, K, 1.0, A, K, B, N, 0.0, C, N) == sg.ERR_WORKSPACE
    # a shape the kernel does not split needs no workspace: whole-tile kernel
    Z = torch.zeros(1024 * 2048, device=dev)
    print("[gpu] sk unsplit shape without workspace", flush=True)
    assert sg.sgemm_f32_ws_size(v, ROW, 0, 0, 2048, 2048, 64, cus) == (0, 0)
    assert sg.sgemm_f32_variant(v, 2048, 2048, 64, 1.0, Z, 64, Z, 2048, 0.0,
                                torch.empty(2048 * 2048, device=dev), 2048) == 0
    torch.cuda.synchronize()


def test_auto_with_workspace_on_a_split_shape(dev, cus):
    # 3072^3 through sgemm_f32_ws: whatever it picks must match the oracle
    # on every element.
    M = N = K = 3072
    A, B, C0, _, _ = operands(M, N, K, "uniform", 9, 0.0)
    rc, C, wsb = call_sk(None, M, N, K, 1.0, 0.0, A, B, C0, dev, cus, tag="sk-auto")
    assert rc == 0 and wsb > 0
    _, v = sg.sgemm_f32_plan_ws(ROW, 0, 0, M, N, K, 1.0, 0x1000, K, 0x1000, N, 0.0, 0x1000, N,
                                wsb, cus)
    print(f"[gpu] 3072^3 with workspace -> {sg.sgemm_f32_variant_name(v)}", flush=True)
    Cref, babs = oracle.sgemm_ref(A, B, None, 1.0, 0.0)
    rep = check_bound(C, Cref, babs, K)
    print(f"[gpu] 3072^3 with workspace: {rep}", flush=True)
    assert rep.n == M * N
    assert rep.ok, rep
