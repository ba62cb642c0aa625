"""The dispatch model: the library's choice agrees with the tuner's
prediction formula, a model round-trips through the C ABI, bad models are
rejected, and the fit recovers known constants from synthetic timings."""
import random

import pytest

import fp32_gemm_tuning_amd as sg
from fp32_gemm_tuning_amd import tune

P = 0x1000  # aligned placeholder address; planning reads no memory


@pytest.fixture(autouse=True)
def restore_builtin_model():
    yield
    assert sg.sgemm_f32_set_model(None) == 0


def _plan(M, N, K, cus):
    rc, v = sg.sgemm_f32_plan(M, N, K, 1.0, P, K, P, N, 0.0, P, N, cus)
    assert rc == 0
    return sg.sgemm_f32_variant_name(v)


def test_builtin_model_lists_the_tile_kernels_in_order():
    m = sg.sgemm_f32_get_model()
    assert [e["variant"] for e in m] == list(tune.TILE)
    for e in m:
        assert e["overhead_us"] >= 0 and all(0 < x <= 1.5 for x in e["eff"])


def test_library_choice_matches_the_tuner_formula():
    rng = random.Random(7)
    builtin = sg.sgemm_f32_get_model()
    for trial in range(40):
        model = builtin if trial == 0 else [
            {"variant": v, "overhead_us": rng.uniform(0, 30),
             "eff": [rng.uniform(0.3, 1.0) for _ in range(4)]}
            for v in rng.sample(list(tune.TILE), rng.randint(1, len(tune.TILE)))]
        assert sg.sgemm_f32_set_model(model) == 0
        for _ in range(25):
            M, N, K = (rng.choice([64, 100, 257, 1000, 2048, 3000, 4096, 7000]) for _ in range(3))
            cus = rng.choice([1, 80, 256, 304])
            if M <= 32 or M * N * K < 64 * 1024 * 1024:
                continue    # skinny and tiny shapes bypass the model
            assert _plan(M, N, K, cus) == tune.choose(model, M, N, K, cus), (model, M, N, K, cus)


def test_model_round_trip_and_restore():
    m = [{"variant": "mfma_64x64", "overhead_us": 3.0, "eff": [0.5, 0.6, 0.7, 0.8]},
         {"variant": "mfma_128x128", "overhead_us": 12.5, "eff": [0.8, 0.85, 0.9, 0.95]}]
    assert sg.sgemm_f32_set_model(m) == 0
    assert sg.sgemm_f32_get_model() == m
    assert _plan(4096, 4096, 4096, 256) in ("mfma_64x64", "mfma_128x128")
    assert sg.sgemm_f32_set_model([]) == 0
    assert _plan(4096, 4096, 4096, 256) == "mfma_256x256"


@pytest.mark.parametrize("bad", [
    [{"variant": "naive", "overhead_us": 1.0, "eff": [0.5] * 4}],          # not a tiled kernel
    [{"variant": "mfma_64x64", "overhead_us": 1.0, "eff": [0.5] * 4}] * 2,  # repeated
    [{"variant": "mfma_64x64", "overhead_us": -1.0, "eff": [0.5] * 4}],     # negative cost
    [{"variant": "mfma_64x64", "overhead_us": 1.0, "eff": [0.5, 0.0, 0.5, 0.5]}],
    [{"variant": "mfma_64x64", "overhead_us": 1.0, "eff": [0.5, 0.5, 2.0, 0.5]}],
])
def test_bad_models_are_rejected_and_leave_the_model(bad):
    before = sg.sgemm_f32_get_model()
    assert sg.sgemm_f32_set_model(bad) == -3
    assert sg.sgemm_f32_get_model() == before


def test_model_size_limits():
    too_many = [{"variant": "mfma_64x64", "overhead_us": 1.0, "eff": [0.5] * 4}] * 17
    assert sg.sgemm_f32_set_model(too_many) == -2
    lib = sg.lib()
    assert lib.sgemm_f32_set_model(None, 3) == -1
    assert lib.sgemm_f32_get_model(None, 4) == -1
    assert lib.sgemm_f32_get_model(None, 0) == len(tune.TILE)


def test_fit_recovers_synthetic_constants():
    truth = {"mfma_128x128": (11.0, [0.80, 0.87, 0.90, 0.91]),
             "mfma_64x64": (7.5, [0.52, 0.61, 0.69, 0.78])}
    cus = 256
    samples = []
    for (M, N, K) in tune.DEFAULT_SHAPES:
        for v, (t0, eff) in truth.items():
            e = {"variant": v, "overhead_us": t0, "eff": eff}
            samples.append({"variant": v, "M": M, "N": N, "K": K,
                            "ms": tune.predict_us(e, M, N, K, cus) / 1e3})
    model = tune.fit(samples, cus)
    got = {e["variant"]: e for e in model}
    for v, (t0, eff) in truth.items():
        assert abs(got[v]["overhead_us"] - t0) <= 0.5
        for b in range(4):
            assert abs(got[v]["eff"][b] - eff[b]) <= 0.02 * eff[b]
    assert all(r["loss"] == 0.0 for r in tune.check(model, samples, cus))
