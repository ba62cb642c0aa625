"""Planted mistakes in the parity judge must be caught by its pins.

Each case copies oracle/compare.py into a temporary directory, plants one
plausible mistake and runs tests/test_compare_pins.py against the copy in a
child process (ORACLE_COMPARE names it). The pins pass on the real file and
must fail on every mutant.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    # the bound's factor, unit roundoff and growth in K
    "factor_40": ("4.0 * max(int(K), 1) * U32", "40.0 * max(int(K), 1) * U32"),
    "factor_2": ("4.0 * max(int(K), 1) * U32", "2.0 * max(int(K), 1) * U32"),
    "unit_2^-23": ("U32 = 2.0 ** -24", "U32 = 2.0 ** -23"),
    "sqrt_k": ("4.0 * max(int(K), 1) * U32", "4.0 * max(int(K), 1) ** 0.5 * U32"),
    "k_without_floor": ("max(int(K), 1)", "int(K)"),
    "bound_on_largest_babs": ("* U32 * babs", "* U32 * np.max(babs)"),
    # the elementwise comparison
    "strict_compare": ("bad = ~(err <= bnd)", "bad = ~(err < bnd)"),
    "reversed_compare": ("bad = ~(err <= bnd)", "bad = ~(err >= bnd)"),
    "nan_passes": ("bad = ~(err <= bnd)", "bad = err > bnd"),
    # the Frobenius bar
    "frobenius_dropped": ("ok=(n_bad == 0) and (frob <= FROB_BAR)", "ok=(n_bad == 0)"),
    "frobenius_bar_1e-4": ("FROB_BAR = 1e-5", "FROB_BAR = 1e-4"),
    "frobenius_bar_1e-6": ("FROB_BAR = 1e-5", "FROB_BAR = 1e-6"),
    "frobenius_relative_to_c": ("r = np.linalg.norm(Cref.ravel())",
                                "r = np.linalg.norm(C.astype(np.float64).ravel())"),
    # the bit-exact check
    "exact_with_tolerance": ("bad = got.view(np.uint32) != want.view(np.uint32)",
                             "bad = ~(np.abs(got - want) <= 1e-6 * np.abs(want))"),
    "exact_blind_to_zero_sign": ("bad = got.view(np.uint32) != want.view(np.uint32)",
                                 "bad = ~(got == want)"),
    "exact_truncates_reference": ("want = Cref.astype(np.float32)",
                                  "want = np.trunc(Cref * 2.0 ** 23) / 2.0 ** 23\n"
                                  "    want = want.astype(np.float32)"),
    # the mismatch report
    "first_transposed": ("i, j = (int(v) for v in idx[0])", "j, i = (int(v) for v in idx[0])"),
    "first_ignores_sampling": ("gi = int(rows[i]) if rows is not None else i", "gi = i"),
}


def test_pins_pass_on_the_real_file():
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_compare_pins.py")],
        cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "compare.py")).read()
    assert src.count(before) >= 1, f"mutation site for {name} not found"
    path = tmp_path / "compare_mutant.py"
    path.write_text(src.replace(before, after))
    env = dict(os.environ, ORACLE_COMPARE=str(path))
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_compare_pins.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert proc.returncode != 0, f"mutant {name} survived the pins:\n{proc.stdout[-2000:]}"
