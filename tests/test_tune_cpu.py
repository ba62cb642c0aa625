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


def _plan_ws(M, N, K, cus, ws_bytes=1 << 40):
    rc, v = sg.sgemm_f32_plan_ws(sg.ROW_MAJOR, 0, 0, M, N, K, 1.0, P, K, P, N, 0.0, P, N,
                                 ws_bytes, cus)
    assert rc == 0
    return sg.sgemm_f32_variant_name(v)


def test_builtin_model_lists_the_tile_kernels_in_order():
    m = sg.sgemm_f32_get_model()
    assert [e["variant"] for e in m] == list(tune.TILE)
    for e in m:
        assert e["overhead_us"] >= 0 and all(0 < x <= 1.5 for x in e["eff"])
        assert 0 < e["fill4"] <= 1.5 and 0 <= e["tile_us"] <= 1e4


def test_library_choice_matches_the_tuner_formula():
    rng = random.Random(7)
    builtin = sg.sgemm_f32_get_model()
    for trial in range(40):
        model = builtin if trial == 0 else [
            {"variant": v, "overhead_us": rng.uniform(0, 30),
             "eff": [rng.uniform(0.3, 1.0) for _ in range(4)], "fill4": rng.uniform(0.3, 1.0),
             "tile_us": rng.choice([0.0, rng.uniform(0, 20)])}
            for v in rng.sample(list(tune.TILE), rng.randint(1, len(tune.TILE)))]
        assert sg.sgemm_f32_set_model(model) == 0
        for _ in range(25):
            M, N, K = (rng.choice([64, 100, 257, 1000, 2048, 3000, 4096, 7000]) for _ in range(3))
            cus = rng.choice([1, 80, 256, 304])
            if M <= 32 or N <= 32 or M * N * K < 64 * 1024 * 1024:
                continue    # few rows or columns and tiny shapes bypass the model
            # odd K or N: 4-byte fills, so each entry's fill4 applies
            vec = tune.packed_vec(M, N, K)
            assert _plan(M, N, K, cus) == tune.choose(model, M, N, K, cus, vec=vec), \
                (model, M, N, K, cus)
            assert _plan_ws(M, N, K, cus) == tune.choose(model, M, N, K, cus, workspace=True,
                                                         vec=vec), (model, M, N, K, cus)


def test_model_round_trip_and_restore():
    m = [{"variant": "mfma_64x64", "overhead_us": 3.0, "eff": [0.5, 0.6, 0.7, 0.8], "fill4": 0.75,
          "tile_us": 2.5},
         {"variant": "mfma_128x128", "overhead_us": 12.5, "eff": [0.8, 0.85, 0.9, 0.95],
          "fill4": 1.0, "tile_us": 0.0}]
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
    [{"variant": "mfma_64x64", "overhead_us": 1.0, "eff": [0.5] * 4, "fill4": 0.0}],
    [{"variant": "mfma_64x64", "overhead_us": 1.0, "eff": [0.5] * 4, "fill4": 1.6}],
    [{"variant": "mfma_64x64", "overhead_us": 1.0, "eff": [0.5] * 4, "tile_us": -0.5}],
    [{"variant": "mfma_64x64", "overhead_us": 1.0, "eff": [0.5] * 4, "tile_us": 2e4}],
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


@pytest.mark.parametrize("tiles,slices,cus", [(576, 192, 256), (144, 192, 256), (300, 7, 256),
                                              (5, 7, 256), (1, 3, 256), (256, 64, 256),
                                              (1000, 313, 304), (3, 1, 256), (17, 1000, 80)])
def test_sk_split_matches_the_library(tiles, slices, cus):
    # The tuner's copy of the split is what the library's plan implies: a
    # stream-K kernel is planned exactly when the split exists, and its
    # busiest share is whole tiles plus at most one run of slices.
    sp = tune.sk_split(tiles, slices, cus)
    R = tiles % cus
    if R == 0:
        assert sp is None
        return
    dp, sk, wgs, upw = sp
    assert dp == tiles - R and sk == R and wgs <= min(cus, 4 * R)
    assert (wgs - 1) * upw < R * slices <= wgs * upw     # every slice in exactly one run
    pieces = [((t + 1) * slices - 1) // upw - (t * slices) // upw + 1 for t in range(R)]
    assert max(pieces) <= -(-wgs // R) + 1                # about four pieces at most


def test_sk_run_touches_at_most_two_tiles():
    # The stream-K kernel computes a run as at most two straight-line pieces
    # (the rest of the tile it starts in, then the start of the next), which
    # holds because a run never has more slices than a tile (upw <= slices,
    # as G >= R). Checked over many splits, with 256 and other unit counts.
    import random
    rng = random.Random(7)
    cases = [(rng.randint(1, 5000), rng.randint(1, 600), rng.choice([80, 104, 256, 304]))
             for _ in range(3000)]
    cases += [(t, s, 256) for t in range(1, 600, 7) for s in (1, 2, 3, 16, 49, 100)]
    for tiles, slices, cus in cases:
        sp = tune.sk_split(tiles, slices, cus)
        if sp is None:
            continue
        _, R, wgs, upw = sp
        assert upw <= slices, (tiles, slices, cus, sp)
        U = R * slices
        for j in range(wgs):
            u0, u1 = j * upw, min((j + 1) * upw, U)
            assert u0 < u1
            assert (u1 - 1) // slices - u0 // slices <= 1, (tiles, slices, cus, j)


def test_stream_k_is_planned_only_with_a_workspace():
    # 3072^3: 576 tiles of 128x128 on 256 units -> 2 whole tiles each + 64
    # split four ways; without a workspace the stream-K kernels are no
    # candidates.
    M = N = K = 3072
    assert not _plan(M, N, K, 256).endswith("_sk")
    _, need = sg.sgemm_f32_ws_size(-1, sg.ROW_MAJOR, 0, 0, M, N, K, 256)
    assert need > 0
    _, need128 = sg.sgemm_f32_ws_size(sg.sgemm_f32_variant_by_name("mfma_128x128_sk"),
                                      sg.ROW_MAJOR, 0, 0, M, N, K, 256)
    assert 0 < need128 <= need
    # 2 partial slots of 128 x 128 floats per stream-K workgroup (256 of them)
    assert need128 == 2 * 256 * 128 * 128 * 4
    # a workspace one byte short of every stream-K kernel's need keeps them out
    got = _plan_ws(M, N, K, 256, ws_bytes=1)
    assert not got.endswith("_sk")
    # 4096^3 splits nothing (256 tiles of 256x256, 1024 of 128x128)
    assert sg.sgemm_f32_ws_size(-1, sg.ROW_MAJOR, 0, 0, 4096, 4096, 4096, 256) == (0, 0)


def test_ws_size_argument_errors():
    f = sg.sgemm_f32_ws_size
    assert f(-2, 0, 0, 0, 8, 8, 8, 256)[0] == sg.ERR_VARIANT
    assert f(len(sg.VARIANTS), 0, 0, 0, 8, 8, 8, 256)[0] == sg.ERR_VARIANT
    assert f(-1, 2, 0, 0, 8, 8, 8, 256)[0] == -13
    assert f(-1, 0, 3, 0, 8, 8, 8, 256)[0] == -14
    assert f(-1, 0, 0, 3, 8, 8, 8, 256)[0] == -15
    assert f(-1, 0, 0, 0, -1, 8, 8, 256)[0] == -1
    assert f(-1, 0, 0, 0, 8, -1, 8, 256)[0] == -2
    assert f(-1, 0, 0, 0, 8, 8, -1, 256)[0] == -3
    assert f(-1, 0, 0, 0, 0, 8, 8, 256) == (0, 0)
    assert sg.lib().sgemm_f32_ws_size(-1, 0, 0, 0, 8, 8, 8, 256, None) == -12
    # a non-stream-K variant needs nothing
    assert f(sg.sgemm_f32_variant_by_name("mfma_128x128"), 0, 0, 0, 3072, 3072, 3072, 256) == (0, 0)


def test_workspace_argument_checks():
    # NULL or misaligned workspace with a nonzero size: -16, before any launch
    a = (sg.ROW_MAJOR, 0, 0, 64, 64, 64, 1.0, P, 64, P, 64, 0.0, P, 64)
    assert sg.sgemm_f32_ws(*a, 0, 1024, stream=0) == -16
    assert sg.sgemm_f32_ws(*a, P + 4, 1024, stream=0) == -16
    assert sg.sgemm_f32_variant_ws(0, *a, P + 8, 1024, stream=0) == -16
    assert "workspace" in sg.sgemm_f32_strerror(-16)
    assert "workspace" in sg.sgemm_f32_strerror(sg.ERR_WORKSPACE)


def test_fit_recovers_synthetic_constants():
    truth = {"mfma_128x128": (11.0, [0.80, 0.87, 0.90, 0.91], 0.70, 3.5),
             "mfma_64x64": (7.5, [0.52, 0.61, 0.69, 0.78], 0.86, 0.0)}
    cus = 256
    samples = []
    assert any(not tune.packed_vec(*s) for s in tune.DEFAULT_SHAPES)
    for (M, N, K) in tune.DEFAULT_SHAPES:
        vec = tune.packed_vec(M, N, K)
        for v, (t0, eff, f4, tt) in truth.items():
            e = {"variant": v, "overhead_us": t0, "eff": eff, "fill4": f4, "tile_us": tt}
            samples.append({"variant": v, "M": M, "N": N, "K": K, "vec": vec,
                            "ms": tune.predict_us(e, M, N, K, cus, vec) / 1e3})
    model = tune.fit(samples, cus)
    got = {e["variant"]: e for e in model}
    for v, (t0, eff, f4, tt) in truth.items():
        assert abs(got[v]["overhead_us"] - t0) <= 0.5
        assert abs(got[v]["tile_us"] - tt) <= 0.5
        assert abs(got[v]["fill4"] - f4) <= 0.02
        for b in range(4):
            assert abs(got[v]["eff"][b] - eff[b]) <= 0.02 * eff[b]
    assert all(r["loss"] == 0.0 for r in tune.check(model, samples, cus))


def test_tile_geometry_matches_the_library():
    # The tuner's block tiles and stream-K slices are the ones the library
    # was compiled with (sgemm_f32_variant_tile); every other variant
    # reports no tile.
    for i, name in enumerate(sg.VARIANTS):
        rc, bm, bn, bk = sg.sgemm_f32_variant_tile(i)
        if name in tune.TILE:
            assert (rc, bm, bn) == (1, *tune.TILE[name]), name
            if name in tune.SK_BK:
                assert bk == tune.SK_BK[name], name
        else:
            assert (rc, bm, bn, bk) == (0, 0, 0, 0), name
    assert sg.sgemm_f32_variant_tile(-1)[0] == sg.ERR_VARIANT
    assert sg.sgemm_f32_variant_tile(len(sg.VARIANTS))[0] == sg.ERR_VARIANT


@pytest.mark.parametrize("variant", sorted(tune.SK_BK))
@pytest.mark.parametrize("M,N,K", [(3072, 3072, 3072), (1000, 1531, 777), (5000, 5000, 5000),
                                   (2176, 2176, 250), (4096, 4096, 4096), (128, 128, 48)])
def test_library_split_matches_the_tuner(variant, M, N, K):
    # The workspace the library asks for is what the tuner's copy of the split
    # (block tile and K slice per stream-K kernel) implies, so the model's
    # busiest-unit share and the kernel's real split agree.
    bm, bn = tune.TILE[variant]
    sp = tune.sk_split(-(-M // bm) * -(-N // bn), -(-K // tune.SK_BK[variant]), 256)
    want = 0 if sp is None else 2 * sp[2] * bm * bn * 4
    v = sg.sgemm_f32_variant_by_name(variant)
    assert sg.sgemm_f32_ws_size(v, sg.ROW_MAJOR, 0, 0, M, N, K, 256) == (0, want)
