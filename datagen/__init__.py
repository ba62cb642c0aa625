"""Seeded synthetic inputs for the FP32 SGEMM workloads.

This module holds no GEMM arithmetic. It only draws the operand matrices
(A, B and the initial C) and records the workload table, so that the CPU
oracle and the GPU library can be fed identical inputs without sharing any
code that computes the product.

Workloads follow the shapes the source pages measure on (square sizes from
256 up to 8192 and the 4092 size just under a 128-tile multiple, from
"GEMM from scratch", Module 01 "The Numbers"; sizes around tile boundaries
from "Optimizing Matrix Multiply on CUDA, Part 1", section "Small and Odd
Sizes") plus an odd-edged shape and a skinny near-GEMV shape ("GEMM from
scratch", Module 08, "The Regime That Runs LLM Inference").

Value recipes (the pages only say "seeded"; this is the reading used):
  uniform  : 2*U[0,1) - 1 drawn in float32, which lands on multiples of 2^-23
             in [-1, 1) and is exact in FP32.
  normal   : standard normal drawn directly in float32.
  integer  : uniform integers in {-3..3}, stored as float32. Every partial
             sum of a K-term dot product of such values is an integer of
             magnitude <= 9K, so any summation order gives the exact result
             whenever 9K < 2^24.
All draws use numpy's PCG64 generator (``numpy.random.default_rng``).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "HEADLINE",
    "draw",
    "draw_matrix",
    "make_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One SGEMM problem: C = alpha*A*B + beta*C0, row-major, packed strides."""

    name: str
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist: str                 # "uniform" | "normal" | "integer"
    seed_a: int
    seed_b: int
    seed_c: Optional[int]     # None when beta == 0 (C0 is never read)
    description: str

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def bytes_min(self) -> int:
        """Compulsory HBM bytes: read A and B once, write C once, and read C0
        once more when beta != 0."""
        c_passes = 2 if self.beta != 0.0 else 1
        return 4 * (self.M * self.K + self.K * self.N + c_passes * self.M * self.N)

    def integer_variant(self) -> "Workload":
        """Same shape and scalars with {-3..3} entries (seeds + 10)."""
        return dataclasses.replace(
            self,
            name=self.name + "_int",
            dist="integer",
            seed_a=self.seed_a + 10,
            seed_b=self.seed_b + 10,
            seed_c=None if self.seed_c is None else self.seed_c + 10,
            description=self.description + " (integer-valued variant)",
        )


def _w(name, M, N, K, alpha, beta, dist, sa, sb, sc, desc):
    return Workload(name, M, N, K, alpha, beta, dist, sa, sb, sc, desc)


WORKLOADS = {
    w.name: w
    for w in [
        _w("S256", 256, 256, 256, 1.0, 0.0, "uniform", 101, 102, None,
           "square 256^3, alpha=1 beta=0, U[-1,1)"),
        _w("S2048", 2048, 2048, 2048, 1.0, 0.0, "uniform", 201, 202, None,
           "square 2048^3, alpha=1 beta=0, U[-1,1)"),
        _w("S4096", 4096, 4096, 4096, 1.0, 0.0, "uniform", 401, 402, None,
           "square 4096^3, alpha=1 beta=0, U[-1,1)"),
        _w("S4092", 4092, 4092, 4092, 1.0, 0.5, "uniform", 409, 410, 411,
           "square 4092^3 (not a 128 multiple), alpha=1 beta=0.5, U[-1,1)"),
        _w("S8192", 8192, 8192, 8192, 1.0, 0.0, "normal", 801, 802, None,
           "square 8192^3, alpha=1 beta=0, N(0,1)"),
        _w("R_odd", 1000, 1531, 777, 1.0, 0.0, "uniform", 1001, 1002, None,
           "odd edges (1000,1531,777), alpha=1 beta=0, U[-1,1)"),
        _w("R_skinny", 16, 8192, 8192, 1.0, 0.0, "uniform", 1601, 1602, None,
           "skinny near-GEMV (16,8192,8192), alpha=1 beta=0, U[-1,1)"),
        # One GPU's share of an 8-way row split (each GPU holds M/8 rows of A
        # and C and all of B; no exchange). Same seeds as the full problem:
        # the generator fills row by row, so A is exactly the first M/8 rows
        # of the full A.
        _w("S4096_M8", 512, 4096, 4096, 1.0, 0.0, "uniform", 401, 402, None,
           "8-way row shard of S4096: (512,4096,4096), alpha=1 beta=0, U[-1,1)"),
        _w("S8192_M8", 1024, 8192, 8192, 1.0, 0.0, "normal", 801, 802, None,
           "8-way row shard of S8192: (1024,8192,8192), alpha=1 beta=0, N(0,1)"),
    ]
}

# The throughput figure is quoted at N = 4096.
HEADLINE = "S4096"


def draw(rng: np.random.Generator, shape: Tuple[int, ...], dist: str) -> np.ndarray:
    """Draw a float32 array of ``shape`` from one of the recipes above."""
    if dist == "uniform":
        return (np.float32(2.0) * rng.random(shape, dtype=np.float32)) - np.float32(1.0)
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "integer":
        return rng.integers(-3, 4, size=shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def draw_matrix(seed: int, rows: int, cols: int, dist: str, ld: Optional[int] = None,
                pad_value: float = np.nan) -> np.ndarray:
    """A rows x cols matrix in a row-major buffer of leading dimension ``ld``.

    Returns the full (rows, ld) float32 buffer. Columns ``cols..ld-1`` are
    padding filled with ``pad_value`` (NaN by default) so that a kernel that
    reads past a row's end poisons its result.
    """
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("ld must be >= cols")
    rng = np.random.default_rng(seed)
    vals = draw(rng, (rows, cols), dist)
    if ld == cols:
        return np.ascontiguousarray(vals)
    buf = np.full((rows, ld), pad_value, dtype=np.float32)
    buf[:, :cols] = vals
    return buf


def make_inputs(w: Workload, lda: Optional[int] = None, ldb: Optional[int] = None,
                ldc: Optional[int] = None):
    """(A, B, C0) buffers for workload ``w``; C0 is NaN-filled when beta == 0
    so that a kernel reading it when it must not is caught."""
    A = draw_matrix(w.seed_a, w.M, w.K, w.dist, lda)
    B = draw_matrix(w.seed_b, w.K, w.N, w.dist, ldb)
    ldc_ = w.N if ldc is None else ldc
    if w.seed_c is None:
        C0 = np.full((w.M, ldc_), np.nan, dtype=np.float32)
    else:
        C0 = draw_matrix(w.seed_c, w.M, w.N, w.dist, ldc)
    return A, B, C0
