"""Fit sgemm_f32's dispatch model to the device at hand.

The library chooses among its tiled matrix-core kernels with a model of each
kernel's time (include/sgemm_f32.h, sgemm_f32_model_entry): a fixed cost plus
the busiest compute unit's work at a fraction of its peak that depends on how
many tiles that unit holds. This follows the pages' kernel selection by the
busiest SM's work ("Optimizing Matrix Multiply on CUDA, Part 2", "Selecting
Among Three Kernels") and their remark that tile choices do not carry over
between GPUs ("GEMM from scratch", Module 08): the constants are measured.

    measure()  interleaved HIP-event timing of every tiled kernel on a set of
               shapes (the order of kernels rotates between rounds)
    fit()      per kernel, the fixed cost on a grid and, for each tiles-per-CU
               bucket, the median fraction of peak; the fixed cost that best
               predicts that kernel's times (mean |log(predicted/measured)|) wins
    install()  hand a model to the library (sgemm_f32_set_model)
    save(), load()  a model as JSON

Command line (on the GPU):
    python -m fp32_gemm_tuning_amd.tune --out model.json [--quick]
    python -m fp32_gemm_tuning_amd.tune --load model.json   (installs and prints plans)
"""
from __future__ import annotations

import argparse
import json
import math
import random
import sys
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import fp32_gemm_tuning_amd as sg

# Block tile of every kernel the model can choose (the library checks the
# same list when a model is installed), in the built-in model's order, which
# is also the order of preference when predictions tie.
TILE: Dict[str, Tuple[int, int]] = {
    "mfma_128x128": (128, 128),
    "mfma_256x256": (256, 256),
    "mfma_64x128": (64, 128),
    "mfma_64x64": (64, 64),
    "mfma_64x128_kg4": (64, 128),
    "mfma_64x96_kg4": (64, 96),
    "mfma_96x64_kg4": (96, 64),
    "mfma_128x128_kg4": (128, 128),
    "mfma_128x128_sk": (128, 128),
    "mfma_64x128_sk": (64, 128),
    "mfma_256x256_sk": (256, 256),
    "mfma_direct": (32, 32),
}
# Stream-K kernels and their K slice: their busiest unit holds floor(T/C)
# whole tiles plus one run of slices (sk_split in the library), and they are
# candidates only with a workspace, on shapes they split.
SK_BK: Dict[str, int] = {"mfma_128x128_sk": 32, "mfma_64x128_sk": 32, "mfma_256x256_sk": 16}
PEAK_PER_CU = 4 * 64 * 2.4e9   # FP32 matrix FLOP/s of one MI355X compute unit

# Shapes a fit times: square, flat, tall, odd, short-K, the two 8-way row
# shards of 4096^3 and 8192^3 (the 30 the built-in model's tile-kernel rows
# were fitted on), and five where the direct kernel's 32x32 grid holds one or
# two tiles per compute unit.
DEFAULT_SHAPES: List[Tuple[int, int, int]] = [
    (512, 512, 512), (768, 768, 768), (1024, 1024, 1024), (1280, 1280, 1280),
    (1536, 1536, 1536), (2048, 2048, 2048), (2560, 2560, 2560), (3072, 3072, 3072),
    (3584, 3584, 3584), (4096, 4096, 4096), (5000, 5000, 5000), (6144, 6144, 6144),
    (8192, 8192, 8192), (1000, 1531, 777), (1024, 1536, 768), (1000, 1531, 1500),
    (2000, 1531, 777), (8192, 1024, 8192), (4096, 2048, 4096), (1024, 8192, 1024),
    (3000, 3000, 500), (500, 3000, 3000), (4000, 4000, 256), (2048, 2048, 8192),
    (1024, 1024, 4096), (2048, 4096, 2048), (1531, 1000, 777), (2050, 2050, 2050),
    (512, 4096, 4096), (1024, 8192, 8192),
    # where the direct kernel's 32x32 grid holds one or two tiles per unit
    (448, 448, 448), (512, 512, 2048), (256, 1024, 1024), (640, 640, 640), (600, 600, 1200),
]
QUICK_SHAPES: List[Tuple[int, int, int]] = [
    (1024, 1024, 1024), (1000, 1531, 777), (2048, 2048, 2048), (3072, 3072, 3072),
    (4096, 4096, 4096), (8192, 1024, 8192),
]


def packed_vec(M: int, N: int, K: int) -> bool:
    """Whether a packed row-major product (lda = K, ldb = N, 16-byte aligned
    bases) lets the tile kernels fill with 16-byte loads (the library's
    vec_ok); otherwise the model applies the kernel's fill4 factor."""
    return K % 4 == 0 and N % 4 == 0


def bucket(n: float) -> int:
    """Tiles-per-CU bucket of a model entry: n = 1, 2, 3-4, >= 5 (a
    fractional stream-K share counts as its ceiling)."""
    n = math.ceil(n)
    return 0 if n <= 1 else 1 if n == 2 else 2 if n <= 4 else 3


def sk_split(tiles: int, slices: int, num_cus: int) -> Optional[Tuple[int, int, int, int]]:
    """(dp_tiles, sk_tiles, sk_wgs, upw) as the library splits, or None
    when it does not split."""
    cus = max(1, num_cus)
    R = tiles % cus
    if R == 0 or slices < 1 or R * slices > 2**31 - 1:
        return None
    G = min(cus, 4 * R)
    U = R * slices
    upw = -(-U // G)
    return tiles - R, R, -(-U // upw), upw


def tiles_per_cu(variant: str, M: int, N: int, num_cus: int, K: int = 0) -> float:
    """Tiles' worth of work on the busiest compute unit (0 for a stream-K
    kernel that would not split the shape)."""
    bm, bn = TILE[variant]
    tiles = -(-M // bm) * -(-N // bn)
    cus = max(1, num_cus)
    if variant in SK_BK:
        sp = sk_split(tiles, -(-K // SK_BK[variant]), cus)
        if sp is None:
            return 0.0
        return sp[0] // cus + sp[3] / -(-K // SK_BK[variant])
    return float(-(-tiles // cus))


def predict_us(entry: dict, M: int, N: int, K: int, num_cus: int, vec: bool = True,
               peak_per_cu: float = PEAK_PER_CU) -> float:
    """The library's prediction for one model entry (sgemm_f32_model_entry);
    `vec`: the operands take 16-byte fills (else fill4 scales eff)."""
    bm, bn = TILE[entry["variant"]]
    n = tiles_per_cu(entry["variant"], M, N, num_cus, K)
    if n <= 0:
        return math.inf
    eff = entry["eff"][bucket(n)] * (1.0 if vec else entry.get("fill4", 1.0))
    return (entry["overhead_us"] + math.ceil(n) * entry.get("tile_us", 0.0) +
            1e6 * n * 2.0 * bm * bn * K / (peak_per_cu * eff))


def auto_ok(variant: str, M: int, N: int, K: int, vec: bool = True) -> bool:
    """Whether the library's automatic choice may launch `variant` for a
    packed row-major call: not when the kernel instance it would take spills
    registers (4-byte fills of the 256x256 tile, masked or 4-byte fills of
    its stream-K form, 4-byte fills of the 64x128 stream-K kernel, which it
    takes only when the register-staged 16-byte fill cannot run: a
    contiguous extent below 4 or offsets past 2^31 bytes)."""
    if variant == "mfma_256x256":
        return vec
    if variant == "mfma_256x256_sk":
        return vec and M % 256 == 0 and N % 256 == 0 and K % SK_BK[variant] == 0
    if variant == "mfma_64x128_sk":
        fillu = (K >= 4 and N >= 4 and (63 * K + K) * 4 < 2**31
                 and (31 * N + N) * 4 < 2**31)
        return vec or fillu
    return True


def choose(model: Sequence[dict], M: int, N: int, K: int, num_cus: int,
           workspace: bool = False, vec: bool = True) -> str:
    """The entry with the smallest prediction (earlier entries win ties);
    stream-K entries only with a workspace and on shapes they split; no entry
    whose instance for the call would spill (auto_ok); mfma_128x128 when no
    entry applies."""
    best, best_us = None, 0.0
    for e in model:
        if e["variant"] in SK_BK and not workspace:
            continue
        if not auto_ok(e["variant"], M, N, K, vec):
            continue
        us = predict_us(e, M, N, K, num_cus, vec)
        if us == math.inf:
            continue
        if best is None or us < best_us:
            best, best_us = e["variant"], us
    return "mfma_128x128" if best is None else best


def measure(shapes: Iterable[Tuple[int, int, int]], variants: Optional[Sequence[str]] = None,
            rounds: int = 3, calls: int = 4, device=None, log=None) -> List[dict]:
    """Median HIP-event time of each (kernel, shape), kernels interleaved.
    Returns samples {variant, M, N, K, ms}; kernels that reject a shape, and
    stream-K kernels on shapes they do not split, are left out."""
    import torch
    dev = torch.device("cuda:0") if device is None else device
    stream = torch.cuda.current_stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    variants = list(TILE) if variants is None else list(variants)
    ids = {v: sg.sgemm_f32_variant_by_name(v) for v in variants}
    out = []
    for (M, N, K) in shapes:
        g = torch.Generator(device=dev).manual_seed(M * 7 + N * 13 + K)
        A = torch.rand(M, K, device=dev, generator=g) * 2 - 1
        B = torch.rand(K, N, device=dev, generator=g) * 2 - 1
        C = torch.empty(M, N, device=dev)
        _, wsb = sg.sgemm_f32_ws_size(-1, sg.ROW_MAJOR, 0, 0, M, N, K, cus)
        ws = torch.empty(max(16, wsb), dtype=torch.uint8, device=dev)

        def call(v):
            return sg.sgemm_f32_variant_ws(ids[v], sg.ROW_MAJOR, 0, 0, M, N, K, 1.0, A, K, B, N,
                                           0.0, C, N, ws, wsb, stream.cuda_stream)
        times = {v: [] for v in variants}
        ok = {}
        for v in variants:    # first call of each kernel: warm-up and support check
            ok[v] = call(v) == 0 and tiles_per_cu(v, M, N, cus, K) > 0
        torch.cuda.synchronize()
        live = [v for v in variants if ok[v]]
        for r in range(rounds):
            order = live[r % max(1, len(live)):] + live[:r % max(1, len(live))]
            for v in order:
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(calls)]
                for a, b in ev:
                    a.record(stream)
                    call(v)
                    b.record(stream)
                torch.cuda.synchronize()
                times[v] += [a.elapsed_time(b) for a, b in ev]
        for v in live:
            ts = sorted(times[v])
            ms = ts[len(ts) // 2]
            out.append({"variant": v, "M": M, "N": N, "K": K, "ms": ms,
                        "vec": packed_vec(M, N, K)})
            if log:
                log(f"{M}x{N}x{K} {v}: {ms:.4f} ms, {2.0 * M * N * K / ms / 1e9:.1f} TFLOP/s")
        del A, B, C, ws
    return out


def fit(samples: Sequence[dict], num_cus: int, peak_per_cu: float = PEAK_PER_CU,
        t0_grid_us: Optional[Sequence[float]] = None,
        tile_grid_us: Optional[Sequence[float]] = None,
        fill4_grid: Optional[Sequence[float]] = None) -> List[dict]:
    """Per kernel: fixed cost per call, fixed cost per tile and 4-byte-fill
    factor (all three from grids) and per-bucket fractions of peak (medians
    of the measured fractions once the fixed costs are taken off, those of
    4-byte-fill samples divided by the factor; at most 1), choosing the
    triple whose predictions best match the measured times (mean absolute
    log error). Buckets without samples borrow the nearest filled one; a
    kernel without 4-byte-fill samples keeps fill4 = 1."""
    import numpy as np
    t0s = [0.5 * i for i in range(61)] if t0_grid_us is None else list(t0_grid_us)
    tts = [0.5 * i for i in range(41)] if tile_grid_us is None else list(tile_grid_us)
    # fill4 is searched in [0.7, 1]: a kernel meets only a few 4-byte-fill
    # shapes in a fit, and unbounded it followed two of them down to 0.58,
    # which misranked other shapes by up to 10% on MI355X.
    f4_grid = [0.70 + 0.02 * i for i in range(16)] if fill4_grid is None else list(fill4_grid)
    by_v: Dict[str, List[Tuple[float, float, float, bool]]] = {}
    for s in samples:
        bm, bn = TILE[s["variant"]]
        n = tiles_per_cu(s["variant"], s["M"], s["N"], num_cus, s["K"])
        work_us = 1e6 * n * 2.0 * bm * bn * s["K"] / peak_per_cu   # at 100% of peak
        vec = s.get("vec", packed_vec(s["M"], s["N"], s["K"]))
        by_v.setdefault(s["variant"], []).append((n, work_us, s["ms"] * 1e3, vec))
    model = []
    for v in TILE:
        ds = by_v.get(v)
        if not ds:
            continue
        n = np.array([d[0] for d in ds]); w = np.array([d[1] for d in ds])
        t = np.array([d[2] for d in ds]); vec = np.array([d[3] for d in ds])
        nc = np.ceil(n)
        b = np.array([bucket(x) for x in n])
        filled = sorted(set(b.tolist()))
        near = [min(filled, key=lambda k: (abs(k - q), -k)) for q in range(4)]
        f4s = f4_grid if (~vec).any() else [1.0]
        best = None
        for t0 in t0s:
            for tt in tts:
                rem = t - t0 - nc * tt
                # A fraction of peak above 1 is not physical: such fixed costs
                # are too large, and the capped rate shows it in the error.
                e_raw = np.where(rem > 0, w / np.where(rem > 0, rem, 1.0), 1.0)
                for f4 in f4s:
                    e = np.clip(np.where(vec, e_raw, e_raw / f4), 1e-3, 1.0)
                    med = {q: _middle(e[b == q]) for q in filled}
                    full = [med[near[q]] for q in range(4)]
                    eff = np.array([full[q] for q in b]) * np.where(vec, 1.0, f4)
                    err = float(np.mean(np.abs(np.log((t0 + nc * tt + w / eff) / t))))
                    if best is None or err < best[0]:
                        best = (err, t0, tt, full, f4)
        model.append({"variant": v, "overhead_us": round(best[1], 3), "tile_us": round(best[2], 3),
                      "eff": [round(x, 4) for x in best[3]], "fill4": round(best[4], 4),
                      "fit_error": round(best[0], 4)})
    return model


def _middle(x) -> float:
    """The median as the fit takes it: the middle element of the sorted
    values, the upper of the two middle ones for an even count."""
    xs = sorted(float(v) for v in x)
    return xs[len(xs) // 2]


def check(model: Sequence[dict], samples: Sequence[dict], num_cus: int,
          workspace: bool = True) -> List[dict]:
    """Per shape: the kernel the model picks, the fastest measured one, and
    the time lost (fraction). Without `workspace` the stream-K kernels are
    left out of both."""
    by_shape: Dict[Tuple[int, int, int], Dict[str, float]] = {}
    for s in samples:
        if workspace or s["variant"] not in SK_BK:
            by_shape.setdefault((s["M"], s["N"], s["K"]), {})[s["variant"]] = s["ms"]
    res = []
    for (M, N, K), d in by_shape.items():
        sub = [e for e in model if e["variant"] in d]
        pick = choose(sub, M, N, K, num_cus, workspace=workspace, vec=packed_vec(M, N, K))
        fastest = min(d, key=d.get)
        res.append({"shape": [M, N, K], "picked": pick, "fastest": fastest,
                    "loss": round(d[pick] / d[fastest] - 1.0, 4)})
    return res


def install(model: Sequence[dict]) -> int:
    """Hand the model to the library; returns its status code."""
    return sg.sgemm_f32_set_model([{"variant": e["variant"], "overhead_us": e["overhead_us"],
                                    "eff": e["eff"], "fill4": e.get("fill4", 1.0),
                                    "tile_us": e.get("tile_us", 0.0)}
                                   for e in model])


def save(model: Sequence[dict], path: str, meta: Optional[dict] = None) -> None:
    with open(path, "w") as f:
        json.dump({"model": list(model), **(meta or {})}, f, indent=1)


def load(path: str) -> List[dict]:
    with open(path) as f:
        return json.load(f)["model"]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", help="write the fitted model here (JSON)")
    ap.add_argument("--load", help="install a saved model and print the plans of the shapes")
    ap.add_argument("--quick", action="store_true", help="6 shapes instead of 30")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--calls", type=int, default=4)
    ap.add_argument("--random", type=int, default=0, metavar="N",
                    help="N seeded random shapes (sides log-uniform in [300, 6000]) instead")
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--check-installed", action="store_true",
                    help="measure the shapes and report how the installed model (built-in, or "
                         "--load) picks, without fitting: a held-out check")
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("tune needs a GPU", file=sys.stderr)
        return 1
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    shapes = QUICK_SHAPES if args.quick else DEFAULT_SHAPES
    if args.random:
        rng = random.Random(args.seed)
        shapes = [tuple(int(round(math.exp(rng.uniform(math.log(300), math.log(6000)))))
                        for _ in range(3)) for _ in range(args.random)]
    if args.load and args.check_installed:
        rc = install(load(args.load))
        if rc:
            return 1
    elif args.load:
        model = load(args.load)
        rc = install(model)
        print(json.dumps({"installed": args.load, "rc": rc}))
        for (M, N, K) in shapes:
            _, v = sg.sgemm_f32_plan(M, N, K, 1.0, 0x1000, K, 0x1000, N, 0.0, 0x1000, N, cus)
            _, wsb = sg.sgemm_f32_ws_size(-1, sg.ROW_MAJOR, 0, 0, M, N, K, cus)
            _, vw = sg.sgemm_f32_plan_ws(sg.ROW_MAJOR, 0, 0, M, N, K, 1.0, 0x1000, K, 0x1000, N,
                                         0.0, 0x1000, N, wsb, cus)
            print(json.dumps({"shape": [M, N, K], "plan": sg.sgemm_f32_variant_name(v),
                              "plan_with_workspace": sg.sgemm_f32_variant_name(vw),
                              "workspace_bytes": wsb}))
        return 0 if rc == 0 else 1
    samples = measure(shapes, rounds=args.rounds, calls=args.calls,
                      log=lambda m: print(m, file=sys.stderr, flush=True))
    if args.check_installed:
        model = sg.sgemm_f32_get_model()
        out = {"num_cus": cus, "samples": samples}
        for ws in (False, True):
            report = check(model, samples, cus, workspace=ws)
            for r in report:
                print(json.dumps({"workspace": ws, **r}))
            summary = {"workspace": ws, "shapes": len(report),
                       "picked_fastest": sum(r["loss"] == 0.0 for r in report),
                       "worst_loss": max(r["loss"] for r in report),
                       "mean_loss": round(sum(r["loss"] for r in report) / len(report), 4)}
            print(json.dumps(summary))
            out["check_workspace" if ws else "check"] = report
            out["summary_workspace" if ws else "summary"] = summary
        if args.out:
            with open(args.out, "w") as f:
                json.dump(out, f)
        return 0
    model = fit(samples, cus)
    report = check(model, samples, cus)
    for e in model:
        print(json.dumps(e))
    worst = max(r["loss"] for r in report)
    picked_fastest = sum(r["loss"] == 0.0 for r in report)
    print(json.dumps({"shapes": len(report), "picked_fastest": picked_fastest,
                      "worst_loss": worst}))
    if args.out:
        save(model, args.out, {"num_cus": cus, "samples": samples, "check": report})
    return 0


if __name__ == "__main__":
    sys.exit(main())
