"""Pins for the parity judge, oracle/compare.py (CPU only).

compare.py decides every parity test: check_exact (bit for bit against the
oracle's FP64 result rounded to FP32) and check_bound (the elementwise bound
|C - Cref| <= 4 * max(K, 1) * 2^-24 * Babs plus the relative Frobenius error
<= 1e-5). The pages give no tolerance; they check the GPU result against a
double-precision CPU result at every element ("100 Days of GPU, Day 44",
"Five paths, one table"). The bound is this library's reading of that
check: the first-order error of a K-term recursive FP32 dot product with 4x
headroom.

Every expected value below is worked out by hand from that definition, with
inputs chosen so the bound is an exact power of two and the error sits
exactly on it or one FP32 step beyond it. A planted mistake in compare.py
(a wrong factor, unit roundoff or K scaling, a strict or reversed
comparison, NaN passing, a dropped Frobenius bar, a tolerance in the exact
check, a sign-of-zero blind exact check, a transposed mismatch index) fails
at least one of them (tests/test_compare_mutants.py plants each one).

ORACLE_COMPARE, if set, names the compare.py file to test (the mutant runs).
"""
import importlib.util
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_PATH = os.environ.get("ORACLE_COMPARE", os.path.join(ROOT, "oracle", "compare.py"))
_spec = importlib.util.spec_from_file_location("compare_under_test", _PATH)
cmp = importlib.util.module_from_spec(_spec)
sys.modules[_spec.name] = cmp          # dataclasses look the module up by name
_spec.loader.exec_module(cmp)

U = 2.0 ** -24          # FP32 unit roundoff, written out here, not read from the module
F32 = np.float32


def a2(*vals, dtype=np.float64):
    return np.array([list(vals)], dtype=dtype)


# ---------------------------------------------------------------------------
# bound()
# ---------------------------------------------------------------------------
def test_bound_by_hand():
    # 4 * 3 * 2^-24 = 12 / 16777216 = 7.152557373046875e-07 per unit of Babs
    got = cmp.bound(a2(1.0, 2.0, 0.0), 3)
    assert got.tolist() == [[7.152557373046875e-07, 1.430511474609375e-06, 0.0]]
    # K = 16: 4 * 16 * 2^-24 = 2^-18 exactly
    assert cmp.bound(a2(1.0), 16).tolist() == [[2.0 ** -18]]
    # K = 1000 on Babs 0.5: 2000 * 2^-24
    assert cmp.bound(a2(0.5), 1000).tolist() == [[2000.0 / 16777216.0]]


def test_bound_k_zero_is_k_one():
    # K = 0: the result is the single rounding of beta*C0; max(K, 1) keeps the
    # bound at 4 * 2^-24 * |beta*C0| instead of zero.
    assert cmp.bound(a2(3.0), 0).tolist() == [[12.0 * U]]
    assert cmp.bound(a2(3.0), 1).tolist() == [[12.0 * U]]


# ---------------------------------------------------------------------------
# check_bound(): the elementwise bar
# ---------------------------------------------------------------------------
def _one(c, cref, babs, K):
    return cmp.check_bound(a2(c, dtype=F32), a2(cref), a2(babs), K)


def test_error_equal_to_bound_passes_next_float_fails():
    # K = 1, Babs = 1, Cref = 1: bound = 4 * 2^-24 = 2^-22.
    assert (1.0 + 2.0 ** -22) == float(F32(1.0 + 2.0 ** -22))       # representable
    r = _one(1.0 + 2.0 ** -22, 1.0, 1.0, 1)
    assert r.ok and r.n_bad == 0 and r.max_bound_util == 1.0
    # the next FP32 value above (ulp at 1 is 2^-23): error 1.5 * 2^-22
    r = _one(1.0 + 2.0 ** -22 + 2.0 ** -23, 1.0, 1.0, 1)
    assert not r.ok and r.n_bad == 1 and r.max_bound_util == 1.5
    # below Cref (ulp just below 1 is 2^-24): error 2^-22 passes, 1.25 * 2^-22 fails
    assert _one(1.0 - 2.0 ** -22, 1.0, 1.0, 1).ok
    r = _one(1.0 - 2.0 ** -22 - 2.0 ** -24, 1.0, 1.0, 1)
    assert not r.ok and r.max_bound_util == 1.25


def test_bound_grows_linearly_in_k():
    # K = 16: bound = 2^-18; the error 2^-18 passes, one FP32 step more fails.
    assert _one(1.0 + 2.0 ** -18, 1.0, 1.0, 16).ok
    assert not _one(1.0 + 2.0 ** -18 + 2.0 ** -23, 1.0, 1.0, 16).ok
    # K = 4: bound = 2^-20, so the K = 16 error fails there
    assert not _one(1.0 + 2.0 ** -18, 1.0, 1.0, 4).ok
    assert _one(1.0 + 2.0 ** -20, 1.0, 1.0, 4).ok


def test_bound_is_per_element():
    # Babs = (1, 4), K = 1: bounds 2^-22 and 2^-20. An error of 2^-20 passes on
    # the second element and fails on the first.
    cref, babs = a2(1.0, 4.0), a2(1.0, 4.0)
    ok = cmp.check_bound(a2(1.0, 4.0 + 2.0 ** -20, dtype=F32), cref, babs, 1)
    assert ok.ok and ok.max_bound_util == 1.0
    bad = cmp.check_bound(a2(1.0 + 2.0 ** -20, 4.0, dtype=F32), cref, babs, 1)
    assert not bad.ok and bad.n_bad == 1
    assert bad.first[:2] == (0, 0)
    assert bad.first[4] == 2.0 ** -22          # the element's own bound is reported


def test_bound_utilisation_reported():
    # half the bound: utilisation exactly 0.5
    r = _one(1.0 + 2.0 ** -23, 1.0, 1.0, 1)
    assert r.ok and r.max_bound_util == 0.5 and r.max_abs_err == 2.0 ** -23
    # zero bound with zero error: utilisation 0, passes
    r = cmp.check_bound(a2(0.0, dtype=F32), a2(0.0), a2(0.0), 5)
    assert r.ok and r.max_bound_util == 0.0
    # zero bound with any error fails
    r = cmp.check_bound(a2(2.0 ** -40, dtype=F32), a2(0.0), a2(0.0), 5)
    assert not r.ok and math.isinf(r.max_bound_util)


def test_nan_and_inf_fail_and_are_located():
    C = np.ones((3, 4), F32)
    Cref = np.ones((3, 4))
    babs = np.ones((3, 4))
    C[2, 1] = np.nan
    r = cmp.check_bound(C, Cref, babs, 100)
    assert not r.ok and r.n_bad == 1 and r.first[:2] == (2, 1)
    C[2, 1] = 1.0
    C[1, 3] = np.inf
    r = cmp.check_bound(C, Cref, babs, 100)
    assert not r.ok and r.n_bad == 1 and r.first[:2] == (1, 3)


def test_first_mismatch_maps_sampled_rows_and_columns():
    C = np.ones((2, 3), F32)
    C[1, 2] = 2.0
    r = cmp.check_bound(C, np.ones((2, 3)), np.ones((2, 3)), 1, rows=np.array([5, 9]))
    assert r.first[:4] == (9, 2, 2.0, 1.0)
    r = cmp.check_bound(C, np.ones((2, 3)), np.ones((2, 3)), 1, cols=np.array([4, 7, 11]))
    assert r.first[:2] == (1, 11)
    r = cmp.check_exact(C, np.ones((2, 3)), rows=np.array([5, 9]))
    assert r.first[:2] == (9, 2)
    # the first mismatch in row-major order, not the largest
    C = np.ones((3, 3), F32)
    C[0, 2] = 1.5
    C[2, 0] = 9.0
    assert cmp.check_exact(C, np.ones((3, 3))).first[:2] == (0, 2)


# ---------------------------------------------------------------------------
# check_bound(): the Frobenius bar
# ---------------------------------------------------------------------------
def test_frobenius_bar_fails_even_when_every_element_passes():
    # K = 1000: elementwise bound 4000 * 2^-24 = 2.38e-4 on Babs = 1. An error
    # of 1e-4 on all 64 elements passes elementwise, but the relative Frobenius
    # error is 1e-4 > 1e-5.
    n = 64
    Cref, babs = np.ones((1, n)), np.ones((1, n))
    C = np.full((1, n), F32(1.0001), F32)
    r = cmp.check_bound(C, Cref, babs, 1000)
    assert r.n_bad == 0 and not r.ok
    assert abs(r.frob_rel - (float(F32(1.0001)) - 1.0)) < 1e-12
    # 8e-6 relative passes both bars
    C = np.full((1, n), F32(1.0 + 8e-6), F32)
    r = cmp.check_bound(C, Cref, babs, 1000)
    assert r.ok and r.frob_rel < 1e-5
    # 1.2e-5 relative fails the Frobenius bar only
    C = np.full((1, n), F32(1.0 + 1.2e-5), F32)
    r = cmp.check_bound(C, Cref, babs, 1000)
    assert r.n_bad == 0 and not r.ok


def test_frobenius_value_by_hand():
    # ||(0, 2^-20)|| / ||(3, 4)|| = 2^-20 / 5
    r = cmp.check_bound(a2(3.0, 4.0 + 2.0 ** -20, dtype=F32), a2(3.0, 4.0), a2(3.0, 4.0), 1000)
    assert r.frob_rel == (2.0 ** -20) / 5.0
    # zero reference: 0 when C is zero too, infinite otherwise
    assert cmp.check_bound(a2(0.0, dtype=F32), a2(0.0), a2(1.0), 1).frob_rel == 0.0
    r = cmp.check_bound(a2(2.0 ** -30, dtype=F32), a2(0.0), a2(1.0), 1)
    assert math.isinf(r.frob_rel) and not r.ok


# ---------------------------------------------------------------------------
# check_exact()
# ---------------------------------------------------------------------------
def test_exact_equal_passes():
    Cref = np.array([[1.0, -2.5, 0.0, 7.0e6]])
    r = cmp.check_exact(Cref.astype(F32), Cref)
    assert r.ok and r.n_bad == 0 and r.n == 4


def test_exact_one_ulp_fails():
    Cref = np.array([[1.0, 1000.0]])
    C = Cref.astype(F32)
    C[0, 1] = np.nextafter(F32(1000.0), F32(np.inf))
    r = cmp.check_exact(C, Cref)
    assert not r.ok and r.n_bad == 1 and r.first[:2] == (0, 1)
    C = Cref.astype(F32)
    C[0, 0] = np.nextafter(F32(1.0), F32(0.0))
    assert not cmp.check_exact(C, Cref).ok


def test_exact_sign_of_zero_matters():
    # The integer pins make every partial sum exact, so the GPU's zero must
    # carry the sign IEEE arithmetic gives it (e.g. alpha = -1 times +0 is -0).
    r = cmp.check_exact(np.array([[-0.0]], F32), np.array([[0.0]]))
    assert not r.ok and r.n_bad == 1
    r = cmp.check_exact(np.array([[0.0]], F32), np.array([[-0.0]]))
    assert not r.ok
    assert cmp.check_exact(np.array([[-0.0]], F32), np.array([[-0.0]])).ok


def test_exact_rounds_reference_to_nearest_even():
    # 1 + 2^-24 is halfway between 1 and 1 + 2^-23: ties go to the even 1.0.
    assert cmp.check_exact(np.array([[1.0]], F32), np.array([[1.0 + 2.0 ** -24]])).ok
    assert not cmp.check_exact(np.array([[1.0 + 2.0 ** -23]], F32),
                               np.array([[1.0 + 2.0 ** -24]])).ok
    # 1 + 3 * 2^-24 is halfway between 1 + 2^-23 (odd) and 1 + 2^-22 (even).
    assert cmp.check_exact(np.array([[1.0 + 2.0 ** -22]], F32),
                           np.array([[1.0 + 3 * 2.0 ** -24]])).ok
    # just above the halfway point rounds up
    assert cmp.check_exact(np.array([[1.0 + 2.0 ** -23]], F32),
                           np.array([[1.0 + 2.0 ** -24 + 2.0 ** -40]])).ok


def test_exact_nan_fails():
    r = cmp.check_exact(np.array([[np.nan, 1.0]], F32), np.array([[1.0, 1.0]]))
    assert not r.ok and r.n_bad == 1 and r.first[:2] == (0, 0)
