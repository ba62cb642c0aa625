"""Throughput benchmark: FP32 SGEMM GFLOP/s on one MI355X and % of FP32 peak.

One step is one sgemm_f32 call (the whole hot path) on the 4096^3 workload
(alpha = 1, beta = 0, A and B uniform in [-1, 1), seeded), inputs already in
HBM. An untimed clock warm-up (0.5 s of calls by default, stated in the
output), W untimed warm-up steps, then K timed steps between a device
synchronisation on each side; per-step kernel durations come from HIP events
recorded on the launch stream. Prints ONE JSON line.

Extra objects on that line:
  roofline     - the GEMM kernel's achieved FLOP/s (2*M*N*K per launch / mean
                 launch duration from the events) against MI355X's FP32 matrix
                 peak (157.3 TFLOP/s), plus HBM traffic per launch from the
                 committed rocprofv3 counter summary when it was taken on the
                 current kernel source (else null).
  cpu_baseline - the FP64 CPU oracle timed on this host's cores over a bounded
                 sample of the same workload (whole output rows).
  clock        - the shader clock read on the device right before and right
                 after the timed steps (library clock probe), and rocm-smi's
                 clock and power before the warm-up and after the timed steps.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload S4096]
                  [--variant auto|mfma_128x128|...] [--no-cpu-baseline]
  python bench.py --sweep [--workloads ...] [--variants all|none|a,b] [--context] [--layouts]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP32_PEAK_TFLOPS = 157.3        # MI355X dense FP32 matrix peak (one 32x32x2 MFMA / 64 clk / SIMD)
# MI355X FP32 vector peak: 256 CU x 4 SIMD x 32 FMA lanes x 2 FLOP x 2.4 GHz. The kernels are built
# without packed FP32, and plain v_fmac_f32 still runs above half of this (the peak probe and the
# vector-FMA kernel both exceed 78.6 TFLOP/s), so half-rate is no ceiling and the full figure is
# the one to price against.
FP32_VALU_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The files the traffic-measured kernel (the tiled matrix-core kernels of mfma_pipe.hip) is
# compiled from, with the build flags: a change to any of them voids the stored traffic.
KERNEL_SOURCES = ["fp32_gemm_tuning_amd/csrc/mfma_pipe.hip", "fp32_gemm_tuning_amd/csrc/mfma_pipecore.hpp",
                  "fp32_gemm_tuning_amd/csrc/mfma_common.hpp", "fp32_gemm_tuning_amd/csrc/common.hpp",
                  "fp32_gemm_tuning_amd/csrc/kernels.hpp", "fp32_gemm_tuning_amd/build.py"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(variant_name: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None if it
    was taken on other kernel sources, another kernel or another workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != kernel_source_sha():
        return None
    if rec.get("kernel") != variant_name or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes")


def cpu_baseline(w, A, B, C0, budget_s: float = 12.0):
    """Time the oracle on whole output rows until ~budget_s of CPU work."""
    import numpy as np

    import oracle
    oracle.build(force=False)
    threads = oracle.max_threads()
    chunk = max(threads * 4, 16)
    done, t_total = 0, 0.0
    while done < w.M and t_total < budget_s:
        rows = np.arange(done, min(w.M, done + chunk))
        t0 = time.perf_counter()
        oracle.sgemm_ref_rows(A, B, C0, w.alpha, w.beta, rows)
        t_total += time.perf_counter() - t0
        done += rows.size
        chunk = min(chunk * 2, w.M)
    gflops = 2.0 * done * w.N * w.K / t_total / 1e9
    return {"value": round(gflops, 3), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.M} output rows of {w.name} ({w.M}x{w.N}x{w.K}), "
                      f"FP64 accumulation, {t_total:.1f} s"}


def measured_peaks(dev, stream, cus: int) -> dict:
    """TFLOP/s of the library's peak-rate probes (unpacked FP32 FMA and both
    FP32 MFMA shapes), each timed with HIP events on the launch stream; the
    best of 10 launches (the clock moves between launches of a pure-MFMA
    loop, which draws more power than the GEMM)."""
    import torch

    import fp32_gemm_tuning_amd as sg
    wgs = cus * 8
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    res = {}
    for kind, name, iters in ((0, "valu_fma_f32", 4096), (1, "mfma_f32_32x32x2", 512),
                              (2, "mfma_f32_16x16x4", 512)):
        best = 0.0
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc, flops = sg.sgemm_f32_peak_probe(kind, wgs, iters, out, stream.cuda_stream)
            b.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"peak probe {name} failed: {rc}")
            best = max(best, flops / (a.elapsed_time(b) * 1e-3) / 1e12)
        res[name] = round(best, 2)
    return res


def clock_probe_enqueue(dev, stream, cus: int):
    """Enqueue the library's clock probe on `stream` (no host wait): 4 waves
    of FP32 MFMAs per SIMD, like the GEMM, each workgroup reporting its
    shader-clock and constant-rate counter differences. Called right after
    the timed steps, it runs on the clock they left."""
    import torch

    import fp32_gemm_tuning_amd as sg
    wgs = cus * 4
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    rc, _ = sg.sgemm_f32_peak_probe(3, wgs, 1024, out, stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"clock probe failed: {rc}")
    return out


def clock_probe_read(out) -> dict:
    """Median, min and max over workgroups of the probe's clock, in MHz: the
    ratio of the two counter differences times the constant counter rate."""
    import numpy as np

    import fp32_gemm_tuning_amd as sg
    rc, wall_khz, max_khz = sg.sgemm_f32_clock_rates()
    if rc != 0:
        raise RuntimeError(f"sgemm_f32_clock_rates failed: {rc}")
    v = out.view(-1, 256)[:, :2].cpu().numpy().astype(np.float64)
    mhz = v[:, 0] / v[:, 1] * wall_khz / 1e3
    return {"median": round(float(np.median(mhz)), 1), "min": round(float(mhz.min()), 1),
            "max": round(float(mhz.max()), 1), "max_sclk_mhz": round(max_khz / 1e3, 1)}


def time_calls(call, steps: int, warmup: int, stream):
    """(per-launch durations in ms, timed-region ms) for `steps` calls."""
    import numpy as np
    import torch
    for _ in range(warmup):
        rc = call()
        if rc != 0:
            raise RuntimeError(f"sgemm call failed with {rc}")
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        rc = call()
        ends[i].record(stream)
        if rc != 0:
            raise RuntimeError(f"sgemm call failed with {rc}")
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    return durs, starts[0].elapsed_time(ends[-1])


# Ladder rungs that would take minutes at the largest sizes are timed only on
# the smaller workloads in a sweep.
SLOW_RUNGS = {"naive", "coalesced", "lds_tiled", "reg1d"}
SLOW_OK = {"S256", "R_odd", "R_skinny", "S2048"}


def sweep(args, dev) -> int:
    import torch

    import fp32_gemm_tuning_amd as sg
    from datagen import WORKLOADS, make_inputs
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    names = (list(sg.VARIANTS) if args.variants == "all" else
             [] if args.variants == "none" else args.variants.split(","))
    for wname in args.workloads.split(","):
        w = WORKLOADS[wname]
        A, B, C0 = make_inputs(w)
        dA, dB, dC = (torch.from_numpy(x).to(dev) for x in (A, B, C0))
        if args.context:
            torch.backends.cuda.matmul.allow_tf32 = False
            C1 = dC.clone()

            def ctx():
                if w.beta != 0.0:
                    torch.addmm(C1, dA, dB, beta=w.beta, alpha=w.alpha, out=dC)
                else:
                    torch.mm(dA, dB, out=dC)
                return 0
            if not args.no_clock_warmup:
                clock_warmup(ctx, 0.3)
            durs, _ = time_calls(ctx, args.steps, args.warmup, stream)
            kms = float(durs.mean())
            print(json.dumps({"sweep": True, "workload": wname, "variant": "context:torch.mm fp32",
                              "kernel_ms_mean": round(kms, 4),
                              "kernel_ms_min": round(float(durs.min()), 4),
                              "gflops": round(w.flops / (kms * 1e-3) / 1e9, 1),
                              "pct_fp32_peak": round(100 * w.flops / (kms * 1e-3) / 1e12 /
                                                     FP32_PEAK_TFLOPS, 2),
                              "hbm_gbs_min_bytes": round(w.bytes_min / (kms * 1e-3) / 1e9, 1)}),
                  flush=True)
            del C1
        # Workspace for the stream-K kernels (and for the automatic choice
        # with one, "auto_ws").
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        _, wsb = sg.sgemm_f32_ws_size(-1, sg.ROW_MAJOR, 0, 0, w.M, w.N, w.K, cus)
        ws = torch.empty(max(16, wsb), dtype=torch.uint8, device=dev)
        # Untimed: bring the clock up before the first timed row, so that the
        # rows of a workload compare kernels rather than clock ramps.
        if not args.no_clock_warmup:
            clock_warmup(lambda: sg.sgemm_f32(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta,
                                              dC, w.N, sp))
        for vname in ["auto"] + (["auto_ws"] if args.ws else []) + names:
            if vname in SLOW_RUNGS and wname not in SLOW_OK:
                continue
            if vname == "auto":
                call = lambda: sg.sgemm_f32(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta,
                                            dC, w.N, sp)
                _, vid = sg.sgemm_f32_plan(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta,
                                           dC, w.N, cus)
                label = "auto:" + sg.sgemm_f32_variant_name(vid)
            elif vname == "auto_ws":
                if wsb == 0:
                    continue
                call = lambda: sg.sgemm_f32_ws(sg.ROW_MAJOR, 0, 0, w.M, w.N, w.K, w.alpha, dA, w.K,
                                               dB, w.N, w.beta, dC, w.N, ws, wsb, sp)
                _, vid = sg.sgemm_f32_plan_ws(sg.ROW_MAJOR, 0, 0, w.M, w.N, w.K, w.alpha, dA, w.K,
                                              dB, w.N, w.beta, dC, w.N, wsb, cus)
                label = "auto_ws:" + sg.sgemm_f32_variant_name(vid)
            else:
                vid = sg.sgemm_f32_variant_by_name(vname)
                call = (lambda vid=vid: sg.sgemm_f32_variant_ws(
                    vid, sg.ROW_MAJOR, 0, 0, w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC,
                    w.N, ws, wsb, sp))
                label = vname
            slow = vname in SLOW_RUNGS
            rc = call()
            if rc == sg.ERR_UNSUPPORTED:     # e.g. a 16-byte-load rung on odd leading dims
                print(json.dumps({"sweep": True, "workload": wname, "variant": label,
                                  "skipped": sg.sgemm_f32_strerror(rc)}), flush=True)
                continue
            # Each fast row gets its own untimed warm-up: a row timed right
            # after the slow rungs (or after a kernel that draws less power)
            # otherwise runs part of its calls on a lower clock.
            if not slow and not args.no_clock_warmup:
                clock_warmup(call, 0.15)
            durs, region = time_calls(call, 3 if slow else args.steps,
                                      1 if slow else args.warmup, stream)
            kms = float(durs.mean())
            print(json.dumps({"sweep": True, "workload": wname, "variant": label,
                              "kernel_ms_mean": round(kms, 4),
                              "kernel_ms_min": round(float(durs.min()), 4),
                              "gflops": round(w.flops / (kms * 1e-3) / 1e9, 1),
                              "pct_fp32_peak": round(100 * w.flops / (kms * 1e-3) / 1e12 /
                                                     FP32_PEAK_TFLOPS, 2),
                              "hbm_gbs_min_bytes": round(w.bytes_min / (kms * 1e-3) / 1e9, 1)}),
                  flush=True)
        if args.layouts:
            layout_sweep(w, dA, dB, dC, args, stream)
        del dA, dB, dC, ws
    return 0


def clock_warmup(call, seconds: float = 0.3) -> None:
    """Run `call` back to back, untimed, for about `seconds`."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            call()
        torch.cuda.synchronize()


def layout_sweep(w, dA, dB, dC, args, stream) -> None:
    """The automatic choice through sgemm_f32_ex for every storage order and
    transposition, on buffers of the workload's sizes (each stored operand
    has the same element count in every orientation; leading dimensions are
    the smallest allowed)."""
    import itertools

    import fp32_gemm_tuning_amd as sg
    sp = stream.cuda_stream
    M, N, K = w.M, w.N, w.K
    for layout, ta, tb in itertools.product((sg.ROW_MAJOR, sg.COL_MAJOR), (0, 1), (0, 1)):
        col = layout == sg.COL_MAJOR
        lda = (K if ta else M) if col else (M if ta else K)
        ldb = (N if tb else K) if col else (K if tb else N)
        ldc = M if col else N
        a = (layout, ta, tb, M, N, K, w.alpha, dA, lda, dB, ldb, w.beta, dC, ldc)
        _, vid = sg.sgemm_f32_plan_ex(*a, torch_cus(dA))
        durs, _ = time_calls(lambda: sg.sgemm_f32_ex(*a, sp), args.steps, args.warmup, stream)
        kms = float(durs.mean())
        print(json.dumps({"sweep": True, "workload": w.name,
                          "layout": ("col" if col else "row") + "-" + "NT"[ta] + "NT"[tb],
                          "variant": "auto:" + sg.sgemm_f32_variant_name(vid),
                          "kernel_ms_mean": round(kms, 4),
                          "kernel_ms_min": round(float(durs.min()), 4),
                          "gflops": round(w.flops / (kms * 1e-3) / 1e9, 1),
                          "pct_fp32_peak": round(100 * w.flops / (kms * 1e-3) / 1e12 /
                                                 FP32_PEAK_TFLOPS, 2)}), flush=True)


def torch_cus(t) -> int:
    import torch
    return torch.cuda.get_device_properties(t.device).multi_processor_count


def smi_snapshot() -> dict:
    """Current graphics clock (MHz) from rocm-smi and socket power (W) from
    amd-smi (rocm-smi reports no power on every system), both read-only;
    fields a tool does not report are left out."""
    import subprocess
    res = {}
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"],
                             capture_output=True, text=True, timeout=20).stdout
        card = next(iter(json.loads(out[out.index("{"):]).values()))
        for k, v in card.items():
            kl = k.lower()
            try:
                if kl.startswith("sclk") and "speed" in kl:
                    res["sclk_mhz"] = float(str(v).strip("() ").lower().replace("mhz", ""))
                elif "power" in kl and "(w)" in kl:
                    res["power_w"] = float(v)
            except ValueError:
                pass
    except Exception:
        pass
    if "power_w" not in res:
        try:
            out = subprocess.run(["amd-smi", "metric", "--power", "--json"],
                                 capture_output=True, text=True, timeout=20).stdout
            d = json.loads(out[out.index("{"):])
            gpus = d["gpu_data"] if isinstance(d, dict) else d
            res["power_w"] = float(gpus[0]["power"]["socket_power"]["value"])
        except Exception:
            pass
    return res


def smi_under_load(call, seconds_first: float = 0.3, cap_s: float = 20.0) -> dict:
    """smi_snapshot() read while `call` keeps running back to back (untimed):
    the tools take about a second, and read after a synchronisation they see
    an idle GPU and its idle power. A thread runs the read; this one keeps
    the GPU busy until it returns."""
    import threading
    import torch
    res = {}
    clock_warmup(call, seconds_first)
    th = threading.Thread(target=lambda: res.update(smi_snapshot()), daemon=True)
    th.start()
    t0 = time.perf_counter()
    while th.is_alive() and time.perf_counter() - t0 < cap_s:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    th.join(timeout=1.0)
    return res


def copy_bandwidth_gbs(dev, mib: int = 1024, reps: int = 5) -> float:
    """Best device-to-device copy rate, counting bytes read plus bytes written."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        best = max(best, 2.0 * n * 4 / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    return best


# Workloads timed back to back over one event pair (launch overhead exposed).
B2B_CALLS = {"S256": 200, "R_odd": 200, "R_skinny": 200}


def regimes(args, dev) -> int:
    """Per workload, with the automatic dispatch and inputs resident: per-launch
    event times, back-to-back throughput, the shape's roofline from a measured
    copy bandwidth, clock and power around the timed sets, and the oracle's
    all-core and single-core rates on the small shapes. R_skinny also runs
    cold: its calls alternate between two copies of B (537 MB, more than the
    256 MB last-level cache)."""
    import numpy as np
    import torch

    import fp32_gemm_tuning_amd as sg
    import oracle
    from datagen import WORKLOADS, make_inputs
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    bw = copy_bandwidth_gbs(dev)
    print(json.dumps({"regimes": True, "copy_bandwidth_gbs": round(bw, 1)}), flush=True)
    oracle.build(force=False)
    for wname in args.workloads.split(","):
        w = WORKLOADS[wname]
        A, B, C0 = make_inputs(w)
        dA, dB, dC = (torch.from_numpy(x).to(dev) for x in (A, B, C0))
        cold = wname == "R_skinny"
        dB2 = dB.clone() if cold else None
        _, vid = sg.sgemm_f32_plan(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC, w.N, cus)
        flip = [0]

        def call(bsel=None):
            b = dB if bsel is None else bsel
            return sg.sgemm_f32(w.M, w.N, w.K, w.alpha, dA, w.K, b, w.N, w.beta, dC, w.N, sp)

        def call_cold():
            flip[0] ^= 1
            return call(dB2 if flip[0] else dB)

        ai = w.flops / w.bytes_min
        roof = min(FP32_PEAK_TFLOPS, ai * bw / 1e3)
        rec = {"regimes": True, "workload": wname, "kernel": sg.sgemm_f32_variant_name(vid),
               "ai_flop_per_byte": round(ai, 2), "roofline_tflops": round(roof, 2),
               "roofline_bound": "fp32" if roof >= FP32_PEAK_TFLOPS else "hbm(measured copy)"}
        for tag, fn in (("warm", call), ("cold", call_cold)) if cold else (("warm", call),):
            smi0 = smi_snapshot()
            # The snapshot leaves the GPU idle for about a second; after such a
            # gap the first tens of milliseconds of calls run slower, so warm
            # up by time (untimed) before the timed calls.
            fn()
            clock_warmup(fn, 0.3)
            durs, _ = time_calls(fn, args.steps, args.warmup, stream)
            n_b2b = B2B_CALLS.get(wname, args.steps)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n_b2b):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            smi1 = smi_snapshot()
            b2b = a.elapsed_time(b) / n_b2b
            tf = w.flops / (float(np.median(durs)) * 1e-3) / 1e12
            rec[tag] = {"event_ms_mean": round(float(durs.mean()), 4),
                        "event_ms_median": round(float(np.median(durs)), 4),
                        "event_ms_min": round(float(durs.min()), 4),
                        "b2b_calls": n_b2b, "b2b_ms_per_call": round(b2b, 4),
                        "tflops_median": round(tf, 2),
                        "tflops_b2b": round(w.flops / (b2b * 1e-3) / 1e12, 2),
                        "pct_of_roofline": round(100 * tf / roof, 1),
                        "pct_fp32_peak": round(100 * tf / FP32_PEAK_TFLOPS, 1),
                        "smi_before": smi0, "smi_after": smi1}
        if wname in ("S256", "R_odd"):
            res = {}
            nthreads = oracle.max_threads()
            for th in (nthreads, 1):
                oracle.set_threads(th)
                t0 = time.perf_counter()
                oracle.sgemm_ref(A, B, C0, w.alpha, w.beta)
                res[f"oracle_gflops_{th}_threads"] = round(w.flops / (time.perf_counter() - t0) / 1e9, 2)
            oracle.set_threads(nthreads)
            rec["cpu_oracle"] = res
        print(json.dumps(rec), flush=True)
        del dA, dB, dC, dB2
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 100 untimed steps (about 0.1 s at 4096^3) let the clock ramp up; with 5
    # the timed steps still see the ramp (about 3% lower).
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--clock-warmup-s", type=float, default=0.5,
                    help="untimed seconds of back-to-back calls before the warm-up steps "
                         "(0 to skip); reported in the output line")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time every variant on --workloads (one JSON line each)")
    ap.add_argument("--workloads",
                    default="S256,R_odd,R_skinny,S2048,S4092,S4096,S8192,S4096_M8,S8192_M8")
    ap.add_argument("--variants", default="all",
                    help="comma-separated variant names, 'all', or 'none' (automatic choice only)")
    ap.add_argument("--context", action="store_true",
                    help="in a sweep, also time torch's FP32 matmul (vendor library, "
                         "TF32 off) as context")
    ap.add_argument("--no-clock-warmup", action="store_true",
                    help="in a sweep, skip the untimed clock warm-up before each workload "
                         "(counter runs, which count every dispatch)")
    ap.add_argument("--ws", action="store_true",
                    help="in a sweep, also time the automatic choice with a workspace "
                         "(sgemm_f32_ws, which may pick a stream-K kernel)")
    ap.add_argument("--layouts", action="store_true",
                    help="in a sweep, also time the automatic choice through sgemm_f32_ex "
                         "for row- and column-major storage and every transposition")
    ap.add_argument("--regimes", action="store_true",
                    help="per workload on --workloads: event and back-to-back timing, "
                         "roofline from a measured copy bandwidth, clock/power, oracle "
                         "rates (one JSON line each)")
    ap.add_argument("--peak", action="store_true",
                    help="only run the peak-rate probes and print them")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (a known-size "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this SGEMM runs on a single MI355X; multi-GPU sharding is a design note only)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import fp32_gemm_tuning_amd as sg
    from datagen import HEADLINE, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.calib_copy:
        n = args.calib_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.sweep:
        return sweep(args, dev)
    if args.regimes:
        return regimes(args, dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if args.peak:
        print(json.dumps({"measured_peak_tflops": measured_peaks(dev, torch.cuda.current_stream(dev),
                                                                 cus)}), flush=True)
        return 0
    w = WORKLOADS[args.workload or HEADLINE]
    A, B, C0 = make_inputs(w)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.from_numpy(C0).to(dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    if args.variant == "auto":
        rc, vid = sg.sgemm_f32_plan(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC, w.N, cus)
        assert rc == 0
        call = lambda: sg.sgemm_f32(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC, w.N, sp)
    else:
        vid = sg.sgemm_f32_variant_by_name(args.variant)
        if vid < 0:
            print(f"unknown variant {args.variant}", file=sys.stderr)
            return 2
        call = lambda: sg.sgemm_f32_variant(vid, w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N,
                                            w.beta, dC, w.N, sp)
    vname = sg.sgemm_f32_variant_name(vid)

    smi_before = smi_snapshot()
    # Untimed clock warm-up (stated in the output): a fixed stretch of calls
    # brings the shader clock up from idle, so the timed steps do not depend
    # on how many warm-up steps the caller asked for.
    if args.clock_warmup_s > 0:
        rc = call()
        if rc != 0:
            print(f"sgemm_f32 failed: {rc} {sg.sgemm_f32_strerror(rc)}", file=sys.stderr)
            return 1
        clock_warmup(call, args.clock_warmup_s)
    for _ in range(args.warmup):
        rc = call()
        if rc != 0:
            print(f"sgemm_f32 failed: {rc} {sg.sgemm_f32_strerror(rc)}", file=sys.stderr)
            return 1
    # Both clock probes are read only after the timed steps: a host stall of
    # 10 ms or more between the warm-up and the timed steps (a read-back, say)
    # is followed by about 40 calls that run up to 20% slower while the shader
    # clock reads unchanged, so nothing but a synchronisation separates them.
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    clk_before_out = clock_probe_enqueue(dev, stream, cus)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record(stream)
        rc = call()
        ends[i].record(stream)
        if rc != 0:
            print(f"sgemm_f32 failed: {rc}", file=sys.stderr)
            return 1
    clk_out = clock_probe_enqueue(dev, stream, cus)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0      # includes the clock probe's run (under 1 ms)
    clk_before = clock_probe_read(clk_before_out)
    clk_after = clock_probe_read(clk_out)
    smi_after = smi_snapshot()
    smi_load = smi_under_load(call)
    durs = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])  # ms
    region_ms = starts[0].elapsed_time(ends[-1])
    ms_per_step = region_ms / K
    flops = float(w.flops)
    value = flops / (ms_per_step * 1e-3) / 1e9
    kernel_ms = float(durs.mean())
    achieved_tflops = flops / (kernel_ms * 1e-3) / 1e12
    is_valu = vname in ("naive", "coalesced", "lds_tiled", "reg1d", "reg2d", "vec4_transa",
                        "valu_main")
    peak = FP32_VALU_PEAK_TFLOPS if is_valu else FP32_PEAK_TFLOPS
    traffic = stored_traffic(vname, w.name)

    out = {
        "metric": "FP32 SGEMM GFLOP/s at N=4096 on 1 MI355X; % of FP32 peak",
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"sgemm {w.name} M=N=K={w.M}" if w.M == w.N == w.K else
                   f"sgemm {w.name} M={w.M} N={w.N} K={w.K}",
                   "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
                   "layout": "row-major, packed lda=K ldb=N ldc=N",
                   "inputs": f"{w.dist}, seeds {w.seed_a}/{w.seed_b}",
                   "kernel": vname},
        "pct_of_fp32_peak": round(100.0 * value / 1e3 / FP32_PEAK_TFLOPS, 2),
        "roofline": {"bound": "alu" if is_valu else "mfma",
                     "achieved": round(achieved_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / peak, 4), "traffic": traffic,
                     "kernel_ms_mean": round(kernel_ms, 4),
                     "kernel_ms_min": round(float(durs.min()), 4),
                     "flops_per_launch": int(flops)},
        "wall_s_timed_region": round(wall, 3),
        "clock": {"warmup_untimed_s": args.clock_warmup_s,
                  "sclk_mhz_device_before": clk_before, "sclk_mhz_device_after": clk_after,
                  "smi_before": smi_before, "smi_after": smi_after,
                  "smi_under_load_after": smi_load},
    }
    peaks = measured_peaks(dev, stream, cus)
    mpk = peaks["valu_fma_f32"] if is_valu else peaks["mfma_f32_32x32x2"]
    out["measured_peak_tflops"] = peaks
    out["roofline"]["frac_of_measured_peak"] = round(achieved_tflops / mpk, 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, A, B, C0)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
