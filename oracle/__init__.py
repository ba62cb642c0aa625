"""CPU oracle for FP32 SGEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The GPU library never imports, links or calls
it, and it shares no code with the GPU library; the only common module is
``datagen`` (seeded input generators, no GEMM arithmetic).

The arithmetic lives in ``oracle.c`` (plain C, FP64 accumulation, OpenMP over
rows). This module only marshals numpy arrays into that C library through
ctypes and rounds its double result to float32 when asked.

Definition followed: C = alpha*A*B + beta*C0 on row-major matrices, each
output the K-term dot product of a row of A and a column of B ("GEMM from
scratch", Module 02, "One Thread Per Output"; "Optimizing Matrix Multiply on
CUDA, Part 1", "Counting the Work"), checked in double precision at every
element ("100 Days of GPU, Day 44", "Five paths, one table").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

__all__ = ["build", "open_lib", "sgemm_ref", "sgemm_ref_rows", "sgemm_ref_cols",
           "max_threads", "set_threads", "lib_path"]


def lib_path() -> str:
    return _LIB


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c (or ``src``) into a shared library with gcc, without
    floating-point contraction, with OpenMP."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


_lib = None


def open_lib(path: str):
    """Load an oracle shared library built from oracle.c (or a copy of it)."""
    lib = ctypes.CDLL(path)
    _declare(lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = open_lib(_LIB)
    return _lib


def _declare(lib):
    i64, f32, vp = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    common = [i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64]
    lib.oracle_sgemm_f64.argtypes = common + [vp, vp]
    lib.oracle_sgemm_f64.restype = ctypes.c_int
    lib.oracle_sgemm_f64_rows.argtypes = common + [i64, vp, vp, vp]
    lib.oracle_sgemm_f64_rows.restype = ctypes.c_int
    lib.oracle_sgemm_f64_cols.argtypes = common + [i64, vp, vp, vp]
    lib.oracle_sgemm_f64_cols.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def _buf(x: Optional[np.ndarray], rows: int, cols: int, name: str) -> Tuple[int, int, object]:
    """(pointer, leading dimension, keep-alive) for a row-major float32 matrix.

    ``x`` may be a 2-D view with unit column stride and any row stride (the
    leading dimension), e.g. a column slice of a wider buffer."""
    if x is None:
        return 0, max(1, cols), None
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.shape[0] < rows or x.shape[1] < cols:
        raise ValueError(f"{name} has shape {x.shape}, needs at least ({rows}, {cols})")
    if x.size == 0:                 # numpy gives empty arrays zero strides
        return x.ctypes.data, max(1, cols), x
    if x.strides[1] != 4 or x.strides[0] % 4 != 0 or x.strides[0] < 4 * x.shape[1]:
        # A fresh copy: numpy calls a one-row (or one-column) view C-contiguous
        # whatever its strides, so ascontiguousarray may hand back a row
        # stride below the row length (a transposed (n, 1) column, say).
        x = np.array(x, dtype=np.float32, order="C", copy=True)
    ld = x.strides[0] // 4
    return x.ctypes.data, max(ld, 1), x


def _args(A, B, C0, M, N, K, alpha, beta):
    pa, lda, ka = _buf(A, M, K, "A")
    pb, ldb, kb = _buf(B, K, N, "B")
    pc, ldc, kc = _buf(C0 if beta != 0.0 else None, M, N, "C0")
    keep = (ka, kb, kc)
    return (M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc), keep


def _dims(A, B, M, N, K):
    if M is None:
        M = A.shape[0]
    if K is None:
        K = A.shape[1]
    if N is None:
        N = B.shape[1]
    return int(M), int(N), int(K)


def sgemm_ref(A: np.ndarray, B: np.ndarray, C0: Optional[np.ndarray] = None,
              alpha: float = 1.0, beta: float = 0.0, M: Optional[int] = None,
              N: Optional[int] = None, K: Optional[int] = None,
              with_bound: bool = True, lib=None):
    """FP64 oracle over every element.

    Returns ``(Cref, Babs)`` as float64 (M, N) arrays, where ``Babs`` is
    ``|alpha|*(|A||B|) + |beta|*|C0|`` (None when ``with_bound`` is False).
    ``A``, ``B`` and ``C0`` are row-major float32 arrays whose row strides
    are the leading dimensions; ``M``, ``N``, ``K`` default to their shapes.
    """
    M, N, K = _dims(A, B, M, N, K)
    args, keep = _args(A, B, C0, M, N, K, alpha, beta)
    out = np.empty((M, N), dtype=np.float64)
    babs = np.empty((M, N), dtype=np.float64) if with_bound else None
    rc = (lib or _load()).oracle_sgemm_f64(*args, out.ctypes.data,
                                           babs.ctypes.data if babs is not None else None)
    del keep
    if rc != 0:
        raise ValueError(f"oracle_sgemm_f64 rejected its arguments (rc={rc})")
    return out, babs


def sgemm_ref_rows(A, B, C0, alpha, beta, rows: Sequence[int], M=None, N=None, K=None,
                   lib=None):
    """Oracle on the listed output rows only: (len(rows), N) arrays."""
    M, N, K = _dims(A, B, M, N, K)
    args, keep = _args(A, B, C0, M, N, K, alpha, beta)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((r.size, N), dtype=np.float64)
    babs = np.empty((r.size, N), dtype=np.float64)
    rc = (lib or _load()).oracle_sgemm_f64_rows(*args, r.size, r.ctypes.data,
                                                out.ctypes.data, babs.ctypes.data)
    del keep
    if rc != 0:
        raise ValueError(f"oracle_sgemm_f64_rows rejected its arguments (rc={rc})")
    return out, babs


def sgemm_ref_cols(A, B, C0, alpha, beta, cols: Sequence[int], M=None, N=None, K=None,
                   lib=None):
    """Oracle on the listed output columns only: (M, len(cols)) arrays."""
    M, N, K = _dims(A, B, M, N, K)
    args, keep = _args(A, B, C0, M, N, K, alpha, beta)
    c = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    out = np.empty((M, c.size), dtype=np.float64)
    babs = np.empty((M, c.size), dtype=np.float64)
    rc = (lib or _load()).oracle_sgemm_f64_cols(*args, c.size, c.ctypes.data,
                                                out.ctypes.data, babs.ctypes.data)
    del keep
    if rc != 0:
        raise ValueError(f"oracle_sgemm_f64_cols rejected its arguments (rc={rc})")
    return out, babs
