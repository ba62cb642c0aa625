"""Compile-time autotuner: sweep the tile parameters of the matrix-core kernels.

The pages tune their kernels by sweeping the block tile, the K slice and the
per-thread patch, and find that the best choice differs between GPUs ("GEMM
from scratch", Module 08; "Optimizing Matrix Multiply on CUDA, Part 2",
"Increasing the Outputs per Thread"). Here those parameters are compile-time
macros of the matrix-core sources (csrc/mfma_pipe.hip, csrc/mfma_kgroup.hip),
so a sweep builds one copy of the library per
configuration and times the kernel the configuration changes:

  space "tile" (mfma_128x128): block tile BM x BN, wave tile WM x WN, K
        slice BK, waves per SIMD (occupancy target), tile-grouping band
        GROUP_M (SGEMM_M128_*)
  space "pipe" (mfma_256x256): block and wave tile, BK, LDS stages
        (SGEMM_M256_*)
  (both variants are instances of the pipelined kernel k_mfma_pipe)
  space "kg96" (mfma_64x96_kg4): K slice (SGEMM_KG96_BK)

build (on any machine with hipcc; no GPU):
    python -m fp32_gemm_tuning_amd.autotune build --space tile --out DIR [--jobs N]
  compiles the space's source once per configuration (the other sources are shared
  with the in-tree build), links DIR/<config>/libsgemm_f32.so, and writes
  DIR/manifest.json with each configuration's flags, build status and the
  compiler's register / spill report for its kernel. Configurations that fail
  a kernel's static checks are recorded as not built.

run (on the GPU):
    python -m fp32_gemm_tuning_amd.autotune run --dir DIR [--shapes MxNxK,...]
  loads every built copy in one process. Before timing a copy, it checks the
  copy's kernel bit for bit against the in-tree library on a ragged
  integer-valued problem (any summation order is exact there); a copy that
  differs is reported and not timed. Then it times the copies interleaved
  (median of HIP-event times) on each shape, and writes DIR/results.json and
  a table: per shape, every configuration's TFLOP/s and the best one.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import importlib.util
import itertools
import json
import os
import re
import subprocess
import sys
from typing import Dict, List, Optional, Sequence, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))

# Each space: the variant it changes, the kernel whose resource report
# matters (a pattern of its mangled name, filled in from the configuration),
# and the values of its macros. A parameter written "A,B" sets two
# macros together (a block tile or a wave tile). The first value of each list
# is the in-tree default, so the first configuration is the in-tree build.
SPACES: Dict[str, dict] = {
    "tile": {
        "variant": "mfma_128x128",
        "source": "mfma_pipe.hip",
        "kernel": "k_mfma_pipeILi{SGEMM_M128_BM}ELi{SGEMM_M128_BN}ELi{SGEMM_M128_WM}ELi{SGEMM_M128_WN}E",
        "params": {
            "SGEMM_M128_BM,SGEMM_M128_BN": [(128, 128), (64, 128), (128, 64), (256, 128),
                                            (128, 256)],
            "SGEMM_M128_WM,SGEMM_M128_WN": [(64, 32), (64, 64), (32, 64)],
            "SGEMM_M128_BK": [32, 16],
            "SGEMM_M128_WAVES_PER_EU": [4, 2],
            "SGEMM_M128_GROUP_M": [8],   # 4 and 16 measured within noise of 8
        },
    },
    "pipe": {
        "variant": "mfma_256x256",
        "source": "mfma_pipe.hip",
        "kernel": "k_mfma_pipeILi{SGEMM_M256_BM}ELi{SGEMM_M256_BN}ELi{SGEMM_M256_WM}ELi{SGEMM_M256_WN}E",
        "params": {
            "SGEMM_M256_BM,SGEMM_M256_BN": [(256, 256), (256, 128), (128, 256), (128, 128)],
            "SGEMM_M256_WM,SGEMM_M256_WN": [(64, 64)],
            "SGEMM_M256_BK": [16, 32],
            "SGEMM_M256_STAGES": [2, 3],
            "SGEMM_M256_WPE": [4],
        },
    },
    "kg96": {
        "variant": "mfma_64x96_kg4",
        "source": "mfma_kgroup.hip",
        "kernel": "k_mfma_kgroup",
        "params": {"SGEMM_KG96_BK": [16, 32]},
    },
}

LDS_BYTES = 160 * 1024   # per compute unit on gfx950
DEFAULT_SHAPES = [(4096, 4096, 4096), (2048, 2048, 2048), (3072, 3072, 3072),
                  (8192, 1024, 8192), (1024, 8192, 1024), (1000, 1531, 777)]


def _valid(space: str, c: Dict[str, int]) -> bool:
    """Structural rules the kernels assume (the same ones their static checks
    enforce), plus limits that would only fail at launch: waves per
    workgroup, occupancy and LDS."""
    if space == "tile":
        bm, bn, wm, wn = (c["SGEMM_M128_" + k] for k in ("BM", "BN", "WM", "WN"))
        bk, wpe = c["SGEMM_M128_BK"], c["SGEMM_M128_WAVES_PER_EU"]
        waves = (bm // wm) * (bn // wn) if bm % wm == 0 and bn % wn == 0 else 0
        lds = 2 * (bm + bn) * bk * 4
    elif space == "pipe":
        bm, bn, wm, wn = (c["SGEMM_M256_" + k] for k in ("BM", "BN", "WM", "WN"))
        bk, wpe, stages = c["SGEMM_M256_BK"], c["SGEMM_M256_WPE"], c["SGEMM_M256_STAGES"]
        waves = (bm // wm) * (bn // wn) if bm % wm == 0 and bn % wn == 0 else 0
        lds = stages * (bm + bn) * bk * 4
    else:
        return c["SGEMM_KG96_BK"] in (16, 32)
    if waves == 0 or waves > 16 or wm % 32 or wn % 32:
        return False
    if (bm * bk) % 256 or (bn * bk) % 256:      # whole 16-byte fill pieces
        return False
    if -(-waves // 4) > wpe:                     # one workgroup must fit its SIMDs
        return False
    if lds > LDS_BYTES:
        return False
    # accumulators per lane (32x32 blocks x 16) must leave room for operands
    acc = (wm // 32) * (wn // 32) * 16
    return acc + 48 <= 512 // wpe


def configs(space: str, limit: Optional[int] = None) -> List[Dict[str, int]]:
    """Valid configurations of a space (macro -> value), the in-tree defaults
    first."""
    params = SPACES[space]["params"]
    keys = list(params)
    out = []
    for vals in itertools.product(*(params[k] for k in keys)):
        c: Dict[str, int] = {}
        for k, v in zip(keys, vals):
            names = k.split(",")
            for n, x in zip(names, v if len(names) > 1 else (v,)):
                c[n] = x
        if _valid(space, c):
            out.append(c)
    return out if limit is None else out[:limit]


def config_name(space: str, c: Dict[str, int]) -> str:
    short = {k.split("_", 2)[-1].lower(): v for k, v in c.items()}
    return space + "_" + "_".join(f"{k}{v}" for k, v in short.items())


def kernel_pattern(space: str, c: Dict[str, int]) -> str:
    """The part of the mangled kernel name that picks out the instances a
    configuration builds."""
    return SPACES[space]["kernel"].format(**c)


def flags(c: Dict[str, int]) -> List[str]:
    return [f"-D{k}={v}" for k, v in c.items()]


def _build_module():
    spec = importlib.util.spec_from_file_location("sgemm_f32_build", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _resources(remarks: str, kernel: str) -> Dict[str, int]:
    """Largest VGPR count and scratch bytes over all instances of the kernel
    (16- and 4-byte fills, transposes), from the compiler's resource
    remarks; the 4-byte-fill instances may spill where the timed 16-byte
    ones do not."""
    vgpr = scratch = 0
    current = None
    for ln in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            current = m.group(1)
            continue
        if current is None or kernel not in current:
            continue
        m = re.search(r"VGPRs: (\d+)", ln)
        if m:
            vgpr = max(vgpr, int(m.group(1)))
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m:
            scratch = max(scratch, int(m.group(1)))
    return {"vgpr": vgpr, "scratch": scratch}


def build(space: str, out: str, jobs: int = 4, limit: Optional[int] = None, log=print) -> dict:
    b = _build_module()
    b.build(jobs=jobs)                       # the shared objects, current
    os.makedirs(out, exist_ok=True)
    source = SPACES[space]["source"]
    shared = [os.path.join(b.BUILD, os.path.splitext(s)[0] + ".o") for s in b.SOURCES
              if s != source]

    def one(c):
        name = config_name(space, c)
        d = os.path.join(out, name)
        os.makedirs(d, exist_ok=True)
        src, obj, rc, text, cmd = b._compile(source, d, tuple(flags(c)))
        entry = {"name": name, "space": space, "config": c, "flags": flags(c), "built": rc == 0}
        if rc != 0:
            entry["error"] = [ln for ln in text.splitlines() if "error" in ln][:3]
            return entry
        lib = os.path.join(d, "libsgemm_f32.so")
        r = subprocess.run([b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", lib,
                            obj, *shared], capture_output=True, text=True)
        os.remove(obj)
        entry["built"] = r.returncode == 0
        entry["lib"] = os.path.relpath(lib, out)
        entry.update(_resources(text, kernel_pattern(space, c)))
        return entry

    cs = configs(space, limit)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        entries = list(ex.map(one, cs))
    for e in entries:
        log(f"{e['name']}: {'built' if e['built'] else 'not built'}"
            + (f", {e['vgpr']} VGPRs, {e['scratch']} B scratch" if e["built"] else ""))
    manifest = {"space": space, "variant": SPACES[space]["variant"], "configs": entries}
    with open(os.path.join(out, "manifest.json"), "w") as f:
        json.dump(manifest, f, indent=1)
    return manifest


# --- run (GPU) ---------------------------------------------------------------

def _load(path: str):
    lib = ctypes.CDLL(path)
    i64, f32, vp, ci = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
    lib.sgemm_f32_variant.argtypes = [ci, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp]
    lib.sgemm_f32_variant.restype = ci
    lib.sgemm_f32_variant_by_name.argtypes = [ctypes.c_char_p]
    lib.sgemm_f32_variant_by_name.restype = ci
    return lib


def run(d: str, shapes: Sequence[Tuple[int, int, int]] = DEFAULT_SHAPES, rounds: int = 3,
        calls: int = 4, log=print) -> dict:
    import numpy as np
    import torch
    import fp32_gemm_tuning_amd as sg   # the in-tree library: the reference build
    with open(os.path.join(d, "manifest.json")) as f:
        manifest = json.load(f)
    vname = manifest["variant"].encode()
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    sp = st.cuda_stream
    copies = []
    for e in manifest["configs"]:
        if e.get("built"):
            lib = _load(os.path.join(d, e["lib"]))
            copies.append((e["name"], lib, lib.sgemm_f32_variant_by_name(vname)))
    ref_id = sg.sgemm_f32_variant_by_name(manifest["variant"])

    # bit-exact gate: integer inputs, ragged in every dimension
    M, N, K = 301, 263, 133
    g = torch.Generator(device=dev).manual_seed(7)
    A = torch.randint(-3, 4, (M, K), generator=g, device=dev).float()
    B = torch.randint(-3, 4, (K, N), generator=g, device=dev).float()
    C = torch.empty(M, N, device=dev)
    assert sg.sgemm_f32_variant(ref_id, M, N, K, 1.0, A, K, B, N, 0.0, C, N, sp) == 0
    torch.cuda.synchronize()
    ref = C.clone()
    ok = []
    for name, lib, v in copies:
        C.fill_(float("nan"))
        rc = lib.sgemm_f32_variant(v, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0,
                                   C.data_ptr(), N, sp)
        torch.cuda.synchronize()
        same = rc == 0 and bool(torch.equal(C, ref))
        if not same:
            log(f"{name}: differs from the in-tree library (rc {rc}), not timed")
        else:
            ok.append((name, lib, v))
    results = {"variant": manifest["variant"], "checked": [n for n, _, _ in ok],
               "resources": {e["name"]: {k: e.get(k) for k in ("vgpr", "scratch")}
                             for e in manifest["configs"] if e.get("built")},
               "shapes": []}
    for (M, N, K) in shapes:
        A = torch.rand(M, K, device=dev) - 0.5
        B = torch.rand(K, N, device=dev) - 0.5
        C = torch.empty(M, N, device=dev)
        args = lambda lib, v: lib.sgemm_f32_variant(v, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(),
                                                    N, 0.0, C.data_ptr(), N, sp)
        times = {n: [] for n, _, _ in ok}
        for n, lib, v in ok:
            for _ in range(2):
                args(lib, v)
        torch.cuda.synchronize()
        for r in range(rounds):
            order = ok[r % max(1, len(ok)):] + ok[:r % max(1, len(ok))]
            for n, lib, v in order:
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(calls)]
                for a, b in ev:
                    a.record(st)
                    args(lib, v)
                    b.record(st)
                torch.cuda.synchronize()
                times[n] += [a.elapsed_time(b) for a, b in ev]
        row = {"shape": [M, N, K], "tflops": {}}
        for n in times:
            ms = float(np.median(times[n]))
            row["tflops"][n] = round(2.0 * M * N * K / ms / 1e9, 1)
        if row["tflops"]:
            row["best"] = max(row["tflops"], key=row["tflops"].get)
        results["shapes"].append(row)
        log(json.dumps(row))
        del A, B, C
    with open(os.path.join(d, "results.json"), "w") as f:
        json.dump(results, f, indent=1)
    return results


def _shapes(s: str) -> List[Tuple[int, int, int]]:
    return [tuple(int(x) for x in t.split("x")) for t in s.split(",") if t]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    pb = sub.add_parser("build", help="compile one library copy per configuration (no GPU)")
    pb.add_argument("--space", choices=sorted(SPACES), required=True)
    pb.add_argument("--out", required=True)
    pb.add_argument("--jobs", type=int, default=4)
    pb.add_argument("--limit", type=int, default=None, help="first N configurations only")
    pr = sub.add_parser("run", help="check and time the built copies (GPU)")
    pr.add_argument("--dir", required=True)
    pr.add_argument("--shapes", default=",".join("x".join(map(str, s)) for s in DEFAULT_SHAPES))
    pr.add_argument("--rounds", type=int, default=3)
    pl = sub.add_parser("list", help="print the valid configurations of a space")
    pl.add_argument("--space", choices=sorted(SPACES), required=True)
    args = ap.parse_args(argv)
    if args.cmd == "list":
        for c in configs(args.space):
            print(config_name(args.space, c))
        return 0
    if args.cmd == "build":
        build(args.space, args.out, args.jobs, args.limit)
        return 0
    run(args.dir, _shapes(args.shapes), args.rounds)
    return 0


if __name__ == "__main__":
    sys.exit(main())
