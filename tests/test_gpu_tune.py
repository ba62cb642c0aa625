"""GPU: the tuner measures the tiled kernels on this device, fits a dispatch
model that the library accepts, and sgemm_f32 stays correct under it."""
import numpy as np
import pytest

import oracle
from datagen import WORKLOADS, make_inputs
from oracle.compare import check_bound

torch = pytest.importorskip("torch")
import fp32_gemm_tuning_amd as sg  # noqa: E402
from fp32_gemm_tuning_amd import tune  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    oracle.build(force=False)
    yield torch.device("cuda:0")
    assert sg.sgemm_f32_set_model(None) == 0


def test_tune_fit_install_and_run(dev):
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    shapes = [(1000, 1531, 777), (2048, 2048, 1024)]
    print(f"[gpu] tune measure {shapes}", flush=True)
    samples = tune.measure(shapes, rounds=1, calls=2, device=dev)
    assert {s["variant"] for s in samples} == set(tune.TILE)
    assert all(s["ms"] > 0 for s in samples)
    model = tune.fit(samples, cus)
    assert [e["variant"] for e in model] == list(tune.TILE)
    assert tune.install(model) == 0
    got = sg.sgemm_f32_get_model()
    assert [e["variant"] for e in got] == list(tune.TILE)
    # Under the fitted model the automatic choice is the model's own pick for
    # each shape, and the product is still right.
    w = WORKLOADS["R_odd"]
    A, B, C0 = make_inputs(w)
    _, v = sg.sgemm_f32_plan(w.M, w.N, w.K, w.alpha, 0x1000, w.K, 0x1000, w.N, w.beta, 0x1000,
                             w.N, cus)
    assert sg.sgemm_f32_variant_name(v) == tune.choose(model, w.M, w.N, w.K, cus,
                                                       vec=tune.packed_vec(w.M, w.N, w.K))
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    dC = torch.from_numpy(C0).to(dev)
    print(f"[gpu] R_odd under tuned model with {sg.sgemm_f32_variant_name(v)}", flush=True)
    assert sg.sgemm_f32(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC, w.N) == 0
    torch.cuda.synchronize()
    Cref, babs = oracle.sgemm_ref(A, B, C0, w.alpha, w.beta)
    rep = check_bound(dC.cpu().numpy(), Cref, babs, w.K)
    assert rep.ok, rep
