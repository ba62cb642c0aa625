"""Parity checks of a GPU result against the oracle -- TEST INFRASTRUCTURE ONLY.

Two bars:

* Bit-exact: for integer-valued inputs every partial sum is an exactly
  representable integer (or half-integer with beta = 0.5), so the FP32 result
  must equal the oracle's double result rounded to float32, bit for bit.

* Error bound: for general inputs any summation order is a correct result
  (the pages never fix one), so each element must satisfy
      |C - Cref| <= 4 * max(K, 1) * 2^-24 * Babs
  with Babs = |alpha|*(|A||B|) + |beta|*|C0| from the oracle. 2^-24 is the
  FP32 unit roundoff; K * u is the first-order bound of a K-term recursive
  dot product; the factor 4 is headroom for the alpha and beta roundings and
  for fused multiply-adds. max(K, 1) keeps the bound non-zero when K = 0,
  where the result is the single rounding of beta*C0. The relative Frobenius
  error ||C - Cref||_F / ||Cref||_F is reported next to it (bar 1e-5).

The pages' correctness protocol also asks that a failure names the kernel,
the case, and the row and column of the first mismatch ("100 Days of GPU,
Day 44", "Exercise" / "Check"); ``Report.first`` carries that.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

U32 = 2.0 ** -24
FROB_BAR = 1e-5


def bound(babs: np.ndarray, K: int) -> np.ndarray:
    return 4.0 * max(int(K), 1) * U32 * babs


@dataclasses.dataclass
class Report:
    ok: bool
    kind: str                      # "exact" | "bound"
    n: int                         # elements compared
    n_bad: int
    max_abs_err: float
    max_bound_util: float          # max |C - Cref| / bound (0 where bound == 0 and err == 0)
    frob_rel: float
    first: Optional[Tuple[int, int, float, float, float]]  # (i, j, got, want, bound)

    def __str__(self) -> str:
        s = (f"{self.kind}: {'OK' if self.ok else 'FAIL'} n={self.n} bad={self.n_bad} "
             f"max_abs_err={self.max_abs_err:.3e} bound_util={self.max_bound_util:.3f} "
             f"frob_rel={self.frob_rel:.3e}")
        if self.first is not None:
            i, j, g, w, b = self.first
            s += f" first mismatch at (row {i}, col {j}): got {g!r} want {w!r} bound {b:.3e}"
        return s


def _frob(C: np.ndarray, Cref: np.ndarray) -> float:
    d = np.linalg.norm((C.astype(np.float64) - Cref).ravel())
    r = np.linalg.norm(Cref.ravel())
    if r == 0.0:
        return 0.0 if d == 0.0 else float("inf")
    return float(d / r)


def _first(mask: np.ndarray, C, Cref, bnd, rows=None, cols=None):
    idx = np.argwhere(mask)
    if idx.size == 0:
        return None
    i, j = (int(v) for v in idx[0])
    gi = int(rows[i]) if rows is not None else i
    gj = int(cols[j]) if cols is not None else j
    return (gi, gj, float(C[i, j]), float(Cref[i, j]), float(bnd[i, j]) if bnd is not None else 0.0)


def check_exact(C: np.ndarray, Cref: np.ndarray, rows=None, cols=None) -> Report:
    """C (float32) must equal Cref (float64) rounded to float32, bit for bit."""
    want = Cref.astype(np.float32)
    got = np.asarray(C, dtype=np.float32)
    bad = got.view(np.uint32) != want.view(np.uint32)
    err = np.abs(got.astype(np.float64) - Cref)
    n_bad = int(bad.sum())
    return Report(
        ok=n_bad == 0, kind="exact", n=int(got.size), n_bad=n_bad,
        max_abs_err=float(np.nanmax(err)) if err.size else 0.0,
        max_bound_util=0.0, frob_rel=_frob(got, Cref) if got.size else 0.0,
        first=_first(bad, got, Cref, None, rows, cols))


def check_bound(C: np.ndarray, Cref: np.ndarray, Babs: np.ndarray, K: int,
                rows=None, cols=None) -> Report:
    """Elementwise |C - Cref| <= 4*max(K,1)*2^-24*Babs, plus the Frobenius report."""
    got = np.asarray(C, dtype=np.float32).astype(np.float64)
    bnd = bound(Babs, K)
    err = np.abs(got - Cref)
    bad = ~(err <= bnd)            # NaN counts as bad
    with np.errstate(divide="ignore", invalid="ignore"):
        util = np.where(bnd > 0, err / bnd, np.where(err == 0, 0.0, np.inf))
    n_bad = int(bad.sum())
    frob = _frob(got, Cref) if got.size else 0.0
    return Report(
        ok=(n_bad == 0) and (frob <= FROB_BAR),
        kind="bound", n=int(got.size), n_bad=n_bad,
        max_abs_err=float(np.nanmax(err)) if err.size else 0.0,
        max_bound_util=float(np.nanmax(util)) if util.size else 0.0,
        frob_rel=frob, first=_first(bad, got, Cref, bnd, rows, cols))
