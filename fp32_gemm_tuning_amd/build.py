"""Build libsgemm_f32.so for gfx950 with hipcc (in-tree, no JIT cache).

Each translation unit under csrc/ is compiled to an object in _build/, then
linked into fp32_gemm_tuning_amd/libsgemm_f32.so. Packed FP32 instructions are
disabled for the device code (-packed-fp32-ops). The compiler's per-kernel
resource remarks (VGPRs, AGPRs, spills, LDS, occupancy) are saved to
_build/resource_usage.txt.

Usage:  python fp32_gemm_tuning_amd/build.py [--jobs N]
(run as a file: importing the package loads the library this script builds)
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsgemm_f32.so")
ARCH = os.environ.get("SGEMM_F32_ARCH", "gfx950")

SOURCES = ["api.hip", "ladder.hip", "valu_main.hip", "mfma_pipe.hip", "mfma_kgroup.hip",
           "mfma_small.hip", "peak.hip"]

CXXFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _compile(src: str, build_dir: str = BUILD, extra=(), csrc: str = CSRC) -> tuple:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CXXFLAGS, *extra, "-c", os.path.join(csrc, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, proc.returncode, proc.stdout + proc.stderr, cmd


def build(jobs: int = 4, verbose: bool = False, extra_flags=(), out_lib: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile every source (with `extra_flags`, e.g. -D tile macros) into
    build_dir and link out_lib. Returns out_lib."""
    os.makedirs(build_dir, exist_ok=True)
    objs, remarks = [], []
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_compile, src, build_dir, tuple(extra_flags)) for src in SOURCES]
        for fut in futs:
            src, obj, rc, out, cmd = fut.result()
            # Host-pass warnings about the device-only target feature are noise.
            lines = [ln for ln in out.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in ln]
            remarks.extend(ln for ln in lines if "remark:" in ln)
            errs = [ln for ln in lines if "remark:" not in ln]
            if rc != 0:
                sys.stderr.write("\n".join(errs) + "\n")
                raise RuntimeError(f"hipcc failed on {src}: {' '.join(cmd)}")
            if verbose and errs:
                sys.stderr.write("\n".join(errs) + "\n")
            objs.append(obj)
    with open(os.path.join(build_dir, "resource_usage.txt"), "w") as f:
        f.write("\n".join(remarks) + "\n")
    tmp = out_lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_lib)
    return out_lib


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
