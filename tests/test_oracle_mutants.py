"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle.c into a temporary directory, plants one plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, a
wrong leading dimension, a lower-precision accumulator, a wrong bound), builds
that copy on the CPU and runs tests/test_oracle_pins.py against it in a child
process. The pins pass on the real oracle and must fail on every mutant.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "sign_flip": ("s[jj] += p;", "s[jj] -= p;"),
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k + 1 < K; ++k)"),
    "transposed_b": ("double p = aik * (double)brow[jj];",
                     "double p = aik * (double)B[(jj % (K > 0 ? K : 1)) * ldb + (k % (N > 0 ? N : 1))];"),
    "packed_lda": ("double aik = (double)A[i * lda + k];", "double aik = (double)A[i * K + k];"),
    "float_accumulator": ("s[jj] += p;", "s[jj] = (float)(s[jj] + p);"),
    "dropped_alpha": ("double v = al * s[jj];", "double v = s[jj];"),
    "dropped_beta": ("v += be * c;", ""),
    "reads_c0_when_beta_zero": ("if (beta != 0.0f) {\n            double c", "if (1) {\n            double c"),
    "signed_bound": ("a[jj] += fabs(p);", "a[jj] += p;"),
    "packed_ldc": ("double c = (double)C0[i * ldc + j];", "double c = (double)C0[i * N + j];"),
    "swapped_alpha_beta": ("double al = (double)alpha, be = (double)beta;",
                           "double al = (double)beta, be = (double)alpha;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(before) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(before, after)
    path = tmp_path / "oracle_mutant.c"
    path.write_text(mutated)
    lib = oracle.build(force=True, src=str(path), out=str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, ORACLE_LIB=lib)
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, f"mutant {name} survived the pins:\n{proc.stdout[-2000:]}"
