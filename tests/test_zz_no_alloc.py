"""sgemm_f32_ws_static: the stream-K entry points with the library's fixed
device scratch as the workspace, for callers that cannot allocate.

Each call is checked against the entry point it stands in for, on the same
inputs: the automatic form against sgemm_f32_ws given a caller workspace of
SGEMM_F32_SCRATCH_BYTES (the same plan, so the same kernels: bit for bit),
the forced form against sgemm_f32_variant_ws; and both against the FP64
oracle (integer inputs bit-exact, random inputs within the elementwise
bound). Calls come in pairs, the second on a smaller problem, since the
scratch keeps the previous call's contents.
"""
import numpy as np
import pytest

import oracle
from datagen import draw_matrix
from oracle.compare import check_bound, check_exact

torch = pytest.importorskip("torch")
import fp32_gemm_tuning_amd as sg  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    return torch.device("cuda:0")


def _inputs(M, N, K, dist, seed, beta):
    A = draw_matrix(seed, M, K, dist)
    B = draw_matrix(seed + 1, K, N, dist)
    C0 = draw_matrix(seed + 2, M, N, dist) if beta != 0.0 else np.full((M, N), np.nan, np.float32)
    return A, B, C0


def _call(dev, entry, variant, M, N, K, alpha, beta, A, B, C0, tag):
    """One product through `entry` ("static" or "ws"); returns (rc, C)."""
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.from_numpy(C0).to(dev)
    s = torch.cuda.current_stream()
    print(f"[gpu] no-alloc {tag} entry={entry} variant={variant} M={M} N={N} K={K}", flush=True)
    if entry == "static":
        rc = sg.sgemm_f32_ws_static(variant, sg.ROW_MAJOR, 0, 0, M, N, K, alpha, dA, K, dB, N,
                                    beta, dC, N, s.cuda_stream)
    else:
        ws = torch.full((sg.SCRATCH_BYTES,), 0xFF, dtype=torch.uint8, device=dev)
        if variant < 0:
            rc = sg.sgemm_f32_ws(sg.ROW_MAJOR, 0, 0, M, N, K, alpha, dA, K, dB, N, beta, dC, N,
                                 ws, sg.SCRATCH_BYTES, s.cuda_stream)
        else:
            rc = sg.sgemm_f32_variant_ws(variant, sg.ROW_MAJOR, 0, 0, M, N, K, alpha, dA, K, dB, N,
                                         beta, dC, N, ws, sg.SCRATCH_BYTES, s.cuda_stream)
    torch.cuda.synchronize()
    return rc, dC.cpu().numpy()


def _check_oracle(C, A, B, C0, K, alpha, beta, exact):
    Cref, babs = oracle.sgemm_ref(A, B, C0, alpha, beta)
    rep = check_exact(C, Cref) if exact else check_bound(C, Cref, babs, K)
    print(f"[gpu] {rep}", flush=True)
    return rep


def _plan(M, N, K, ws_bytes):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    P = 1 << 20
    rc, v = sg.sgemm_f32_plan_ws(sg.ROW_MAJOR, 0, 0, M, N, K, 1.0, P, K, P, N, 0.0, P, N,
                                 ws_bytes, cus)
    assert rc == 0
    return sg.sgemm_f32_variant_name(v)


# (M, N, K, alpha, beta, dist): each pair is a larger then a smaller problem;
# every one is split by a stream-K kernel that fits the scratch (3584^3 would
# take mfma_256x256_sk, 128 MiB, with an unlimited workspace).
AUTO_PAIRS = [
    [(3584, 3584, 3584, 1.0, 0.0, "integer"), (1792, 1792, 1792, 1.0, 0.0, "uniform")],
    [(2560, 2560, 2560, 1.5, 0.5, "uniform"), (1536, 1536, 1536, -1.0, 0.25, "integer")],
]


@pytest.mark.parametrize("pair", AUTO_PAIRS, ids=["3584-then-1792", "2560-then-1536"])
def test_automatic_matches_ws_entry_point(dev, pair):
    for i, (M, N, K, alpha, beta, dist) in enumerate(pair):
        name = _plan(M, N, K, sg.SCRATCH_BYTES)
        assert name.endswith("_sk"), name          # the scratch is really used
        A, B, C0 = _inputs(M, N, K, dist, 500 + 7 * i + M, beta)
        rc1, C1 = _call(dev, "static", -1, M, N, K, alpha, beta, A, B, C0, f"auto#{i} {name}")
        rc2, C2 = _call(dev, "ws", -1, M, N, K, alpha, beta, A, B, C0, f"auto#{i} {name}")
        assert rc1 == 0 and rc2 == 0, (sg.sgemm_f32_strerror(rc1), sg.sgemm_f32_strerror(rc2))
        assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), f"{name} {M}x{N}x{K}"
        rep = _check_oracle(C1, A, B, C0, K, alpha, beta, dist == "integer")
        assert rep.ok, f"{name} {M}x{N}x{K}: {rep}"


# (variant, M, N, K): forced stream-K kernels whose workspace fits the scratch,
# a larger then a smaller problem each; and a kernel that takes no workspace.
FORCED_PAIRS = [
    ("mfma_256x256_sk", [(5120, 3328, 512), (1280, 768, 1024)]),
    ("mfma_128x128_sk", [(2560, 2560, 640), (1408, 1152, 320)]),
    ("mfma_64x128_sk", [(2560, 2560, 640), (640, 1152, 1000)]),
    ("mfma_128x128", [(1000, 1531, 777), (300, 260, 100)]),
]


@pytest.mark.parametrize("variant,pair", FORCED_PAIRS, ids=[f[0] for f in FORCED_PAIRS])
def test_forced_matches_variant_ws(dev, variant, pair):
    v = sg.sgemm_f32_variant_by_name(variant)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for i, (M, N, K) in enumerate(pair):
        need = sg.sgemm_f32_ws_size(v, sg.ROW_MAJOR, 0, 0, M, N, K, cus)[1]
        assert need <= sg.SCRATCH_BYTES
        if variant.endswith("_sk"):
            assert need > 0, f"{variant} does not split {M}x{N}x{K}"
        dist = "integer" if i == 0 else "uniform"
        A, B, C0 = _inputs(M, N, K, dist, 900 + M + K, 0.5)
        rc1, C1 = _call(dev, "static", v, M, N, K, 1.0, 0.5, A, B, C0, f"forced#{i}")
        rc2, C2 = _call(dev, "ws", v, M, N, K, 1.0, 0.5, A, B, C0, f"forced#{i}")
        assert rc1 == 0 and rc2 == 0, (sg.sgemm_f32_strerror(rc1), sg.sgemm_f32_strerror(rc2))
        assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32)), f"{variant} {M}x{N}x{K}"
        rep = _check_oracle(C1, A, B, C0, K, 1.0, 0.5, dist == "integer")
        assert rep.ok, f"{variant} {M}x{N}x{K}: {rep}"


def test_too_large_for_the_scratch_is_refused(dev):
    # mfma_256x256_sk on 3584^3 needs 128 MiB of partial tiles: refused before
    # any launch, C untouched.
    v = sg.sgemm_f32_variant_by_name("mfma_256x256_sk")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M = N = K = 3584
    need = sg.sgemm_f32_ws_size(v, sg.ROW_MAJOR, 0, 0, M, N, K, cus)[1]
    assert need > sg.SCRATCH_BYTES
    dA = torch.zeros((M, K), dtype=torch.float32, device=dev)
    dB = torch.zeros((K, N), dtype=torch.float32, device=dev)
    dC = torch.full((M, N), 7.0, dtype=torch.float32, device=dev)
    print(f"[gpu] no-alloc refusal M={M}", flush=True)
    rc = sg.sgemm_f32_ws_static(v, sg.ROW_MAJOR, 0, 0, M, N, K, 1.0, dA, K, dB, N, 0.0, dC, N,
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == sg.ERR_SCRATCH, sg.sgemm_f32_strerror(rc)
    assert bool(torch.all(dC == 7.0))
