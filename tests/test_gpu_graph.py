"""HIP graph capture and concurrent streams.

The library enqueues only kernels on the caller's stream (no memset nodes, no
allocation, no synchronisation), so a call can be captured in a graph and
replayed. Each test replays its graph several times, with eager work and
synchronisations between the replays and the output clobbered before each,
and checks every replay bit for bit against the eager call (the same kernels
on the same inputs give the same bits). Stream-K (sgemm_f32_ws) is captured
too: its two kernels and the workspace they share must replay as well.
Separately, two streams run different products at the same time."""
import numpy as np
import pytest

import oracle
from datagen import draw_matrix
from oracle.compare import check_exact

torch = pytest.importorskip("torch")
import fp32_gemm_tuning_amd as sg  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    return torch.device("cuda:0")


def _operands(M, N, K, seed, dev, dist="uniform"):
    A = torch.from_numpy(draw_matrix(seed, M, K, dist)).to(dev)
    B = torch.from_numpy(draw_matrix(seed + 1, K, N, dist)).to(dev)
    C0 = torch.from_numpy(draw_matrix(seed + 2, M, N, dist)).to(dev)
    return A, B, C0


# (M, N, K, use_workspace, variant): the automatic choice at a few sizes,
# and the stream-K kernels (two kernels per call) with a workspace.
CASES = [
    (1000, 1531, 777, False, None),
    (4096, 4096, 1024, False, None),
    (2560, 2560, 512, True, "mfma_128x128_sk"),
    (640, 384, 200, True, "mfma_64x128_sk"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-{c[4] or 'auto'}")
def test_graph_replays_match_eager(dev, case):
    M, N, K, use_ws, variant = case
    A, B, C0 = _operands(M, N, K, 11 + M, dev)
    C = C0.clone()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    vid = -1 if variant is None else sg.sgemm_f32_variant_by_name(variant)
    wsb = sg.sgemm_f32_ws_size(vid, sg.ROW_MAJOR, 0, 0, M, N, K, cus)[1] if use_ws else 0
    ws = torch.empty(max(16, wsb), dtype=torch.uint8, device=dev)

    def call(stream):
        if variant is None:
            return sg.sgemm_f32_ws(sg.ROW_MAJOR, 0, 0, M, N, K, 1.5, A, K, B, N, 0.5, C, N, ws, wsb,
                                   stream.cuda_stream)
        return sg.sgemm_f32_variant_ws(vid, sg.ROW_MAJOR, 0, 0, M, N, K, 1.5, A, K, B, N, 0.5, C,
                                       N, ws, wsb, stream.cuda_stream)

    print(f"[gpu] graph {case}: eager", flush=True)
    s = torch.cuda.Stream(dev)
    with torch.cuda.stream(s):
        assert call(s) == 0
    torch.cuda.synchronize()
    eager = C.clone()

    print(f"[gpu] graph {case}: capture", flush=True)
    g = torch.cuda.CUDAGraph()
    C.copy_(C0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        rc = call(s)
    assert rc == 0
    torch.cuda.synchronize()
    for r in range(4):
        print(f"[gpu] graph {case}: replay {r}", flush=True)
        C.copy_(C0)                      # beta != 0: each replay starts from C0
        ws.fill_(0xFF)                   # the workspace holds garbage before each replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, eager), f"replay {r} differs from the eager call"
        # eager work between replays, on the default stream
        sg.gemm(A[:64, :64].contiguous(), B[:64, :64].contiguous(),
                torch.empty(64, 64, device=dev))
        torch.cuda.synchronize()
    del g


def test_concurrent_streams(dev):
    # Two different integer products on two streams at once; each must match
    # the oracle exactly.
    cases = [(1500, 700, 900, 3), (800, 1300, 1100, 4)]
    streams = [torch.cuda.Stream(dev) for _ in cases]
    outs = []
    for (M, N, K, seed), s in zip(cases, streams):
        A, B, _ = _operands(M, N, K, seed, dev, "integer")
        C = torch.full((M, N), float("nan"), device=dev)
        outs.append((A, B, C))
    torch.cuda.synchronize()
    print("[gpu] two streams", flush=True)
    for _ in range(3):
        for ((M, N, K, _), s), (A, B, C) in zip(zip(cases, streams), outs):
            with torch.cuda.stream(s):
                assert sg.sgemm_f32(M, N, K, 1.0, A, K, B, N, 0.0, C, N, s.cuda_stream) == 0
    torch.cuda.synchronize()
    for (M, N, K, _), (A, B, C) in zip(cases, outs):
        Cref, _ = oracle.sgemm_ref(A.cpu().numpy(), B.cpu().numpy(), None, 1.0, 0.0)
        rep = check_exact(C.cpu().numpy(), Cref)
        assert rep.ok, rep
