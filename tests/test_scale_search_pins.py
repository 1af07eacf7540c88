"""Pins of the oracle's per-row scale search (Appendix D of the BaKron paper:
absmax / largest code, optionally shrunk by up to a factor of 2 by an MSE
search), against facts fixed independently of its code: reduction to the
plain absmax rule, a hand-derived optimum, exact-grid rows, exact invariances
and a scalar brute force in Python floats."""
import math

import numpy as np
import pytest

import oracle as O


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_no_search_is_absmax_rule(dtype):
    W = np.random.default_rng(0).standard_normal((9, 40)).astype(dtype)
    W[3] = 0.0
    plain = O.row_scales(W, 7, dtype)
    assert np.array_equal(O.row_scales_mse(W, -8, 7, 0, 0.5, dtype), plain)
    assert np.array_equal(O.row_scales_mse(W, -8, 7, 50, 0.0, dtype), plain)
    s = O.row_scales_mse(W, -8, 7, 50, 0.5, dtype)
    assert s[3] == 1.0  # all-zero row keeps scale 1


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_hand_derived_optimum(dtype):
    """Row = one 10 and 1000 ones, alphabet {-8..7}, 101 candidates down to
    half the absmax scale s_max = 10/7. Every candidate lies in [5/7, 10/7],
    where each 1 rounds to code 1 and the 10 to code 7 (10/s >= 7), so the
    error is 1000 (1 - s)^2 + (10 - 7 s)^2, a parabola with its minimum at
    s* = 1070/1049 = 1.02002. The candidates are s_k = s_max (1 - k/200);
    s* sits at k = 57.2, between s_57 = 1.02143 and s_58 = 1.01429, and s_57
    is the closer one, so the search must return s_57."""
    row = np.ones(1001, dtype=dtype)
    row[0] = 10.0
    s = O.row_scales_mse(row[None], -8, 7, 100, 0.5, dtype)[0]
    smax = dtype(10.0) / dtype(7.0)
    expect = dtype(np.float64(smax) * (1.0 - 57 * 0.5 / 100))
    assert s == expect, (s, expect)
    assert abs(float(s) - 1070.0 / 1049.0) < 0.0015


def test_exact_grid_row_is_not_shrunk():
    """A row whose entries are exact multiples (within the alphabet) of
    absmax/hi has zero error at k = 0; every smaller candidate clips the
    absmax entry (its code would exceed hi), so no other candidate is exact."""
    row = np.array([7.0, -7.0, 3.0, 0.0, -2.0, 5.0]) * 0.125
    s = O.row_scales_mse(row[None], -8, 7, 64, 0.5, np.float64)[0]
    assert s == 0.125


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_power_of_two_scaling_is_exact(dtype):
    """Multiplying a row by 2^p multiplies every candidate, every quotient's
    denominator and every error by powers of two exactly, so the chosen scale
    scales by exactly 2^p."""
    W = np.random.default_rng(1).standard_normal((6, 300)).astype(dtype) * dtype(0.02)
    s = O.row_scales_mse(W, -4, 3, 40, 0.5, dtype)
    for p in (-6, 3):
        f = dtype(2.0 ** p)
        s2 = O.row_scales_mse(W * f, -4, 3, 40, 0.5, dtype)
        assert np.array_equal(s2, s * f)


def test_negation_with_symmetric_alphabet():
    W = np.random.default_rng(2).standard_normal((5, 200))
    s = O.row_scales_mse(W, -3, 3, 30, 0.5, np.float64)
    assert np.array_equal(O.row_scales_mse(-W, -3, 3, 30, 0.5, np.float64), s)


def test_search_never_worse_than_absmax():
    W = np.random.default_rng(3).standard_t(4, (20, 256)) * 0.02
    s0 = O.row_scales(W, 7, np.float64)
    s = O.row_scales_mse(W, -8, 7, 100, 0.5, np.float64)
    e0 = O.row_rtn_error(W, s0, -8, 7)
    e = O.row_rtn_error(W, s, -8, 7)
    assert np.all(e <= e0)
    assert np.all(s <= s0) and np.all(s >= 0.5 * s0 * (1 - 1e-15))
    # heavy-tailed rows gain from shrinking
    assert np.mean(e < e0) > 0.5


def test_brute_force_in_python_floats():
    """Scalar re-derivation with Python floats (IEEE double; round() ties to
    even) on small rows: the oracle's choice attains the smallest error of
    all candidates, and no earlier candidate attains it."""
    rng = np.random.default_rng(4)
    for _ in range(30):
        row = [float(x) for x in rng.standard_t(3, 13)]
        lo, hi, grid, ms = -4, 3, 17, 0.5
        smax = max(abs(x) for x in row) / hi
        errs = []
        for k in range(grid + 1):
            sk = smax * (1.0 - ms * k / grid)
            tot = 0.0
            for x in row:
                c = min(max(round(x / sk), lo), hi)
                tot += (x - sk * c) ** 2
            errs.append((tot, sk))
        s = O.row_scales_mse(np.array([row]), lo, hi, grid, ms, np.float64)[0]
        best = min(e for e, _ in errs)
        first = next(sk for e, sk in errs if e == best)
        chosen = [e for e, sk in errs if sk == s]
        assert chosen and math.isclose(chosen[0], best, rel_tol=1e-12)
        assert s == first or math.isclose(chosen[0], best, rel_tol=1e-12)
