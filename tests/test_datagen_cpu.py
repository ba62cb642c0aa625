"""The seeded input recipes: values, ranges and the row-shard property."""
import numpy as np
import pytest

from datagen import WORKLOADS, draw_matrix, make_inputs


@pytest.mark.parametrize("full,shard", [("S4096", "S4096_M8"), ("S8192", "S8192_M8")])
def test_row_shards_are_the_first_rows_of_the_full_problem(full, shard):
    # An 8-way row split gives each GPU M/8 rows of A and all of B; with the
    # same seeds the shard's A is exactly the full A's first rows (the
    # generator fills row by row), checked here on a column slice.
    f, s = WORKLOADS[full], WORKLOADS[shard]
    assert (s.M * 8, s.N, s.K) == (f.M, f.N, f.K)
    assert (s.alpha, s.beta, s.dist, s.seed_a, s.seed_b) == (f.alpha, f.beta, f.dist, f.seed_a, f.seed_b)
    rows = 64
    a_full = draw_matrix(f.seed_a, rows * 8, 32, f.dist)
    a_shard = draw_matrix(s.seed_a, rows, 32, s.dist)
    assert np.array_equal(a_full[:rows], a_shard)


@pytest.mark.parametrize("dist,lo,hi", [("uniform", -1.0, 1.0), ("integer", -3.0, 3.0)])
def test_value_ranges(dist, lo, hi):
    x = draw_matrix(7, 64, 48, dist)
    assert x.dtype == np.float32 and x.shape == (64, 48)
    assert x.min() >= lo and x.max() <= hi
    if dist == "integer":
        assert np.array_equal(x, np.round(x))


def test_padding_is_nan_and_beta_zero_c_is_nan():
    x = draw_matrix(3, 5, 4, "uniform", ld=7)
    assert x.shape == (5, 7) and np.all(np.isnan(x[:, 4:])) and np.all(np.isfinite(x[:, :4]))
    w = WORKLOADS["R_odd"]
    assert w.beta == 0.0
    A, B, C0 = make_inputs(WORKLOADS["S256"])
    assert np.all(np.isnan(C0))
