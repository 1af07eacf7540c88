"""Pins of the oracle's checking helpers: the rounding-midpoint gap, the
replay of recurrence (2) with imposed codes, and the two bounds of
Corollary 3.4 ("BaKron: Efficient Quantization with Kronecker-Factored
Hessians", arXiv 2608.06291; Appendix B for the recurrence, §3.6 for the
corollary). Every expected value below is worked by hand in the docstring or
comment next to it; none is produced by the oracle itself.
"""
import numpy as np
import pytest

import oracle as O


# ------------------------------------------------------------- frac_gap ----

@pytest.mark.parametrize("x,gap", [
    (2.5, 0.0),       # exactly on a midpoint
    (-2.5, 0.0),      # negative midpoint: frac(-2.5) = 0.5
    (2.0, 0.5),       # an integer is half a unit from both midpoints
    (-1.3, 0.2),      # frac(-1.3) = 0.7, |0.7 - 0.5| = 0.2
    (3.75, 0.25),     # frac = 0.75
    (0.1, 0.4),       # frac = 0.1
    (7.0 - 2.0 ** -20, 0.5 - 2.0 ** -20),  # just below an integer
])
def test_frac_gap_hand_values(x, gap):
    assert O.frac_gap(np.float64(x)) == pytest.approx(gap, abs=1e-15)


def test_frac_gap_near_midpoint_is_the_distance():
    # 0.5 + d and 0.5 - d are both d away from the midpoint (d a power of two,
    # so both sums are exact)
    for d in (2.0 ** -10, 2.0 ** -20, 2.0 ** -30):
        assert O.frac_gap(np.float64(4.5 + d)) == d
        assert O.frac_gap(np.float64(-3.5 - d)) == d


# --------------------------------------------------------------- replay ----

def test_replay_single_entry_flags_a_wrong_code_with_its_gap():
    # 1 x 1: the value at rounding is W itself. rint(2.4) = 2; imposing 3 is
    # inconsistent, at |frac(2.4) - 1/2| = 0.1 from the midpoint.
    one = np.ones((1, 1))
    rep = O.replay(np.array([[2.4]]), one, one, (0, 0, 1), O.SCALE_NONE, None, np.array([[3.0]]))
    assert rep.inconsistent == 1
    assert rep.max_inconsistent_gap == pytest.approx(0.1, abs=1e-15)
    assert rep.Wt[0, 0] == 2.4
    ok = O.replay(np.array([[2.4]]), one, one, (0, 0, 1), O.SCALE_NONE, None, np.array([[2.0]]))
    assert ok.inconsistent == 0 and ok.max_inconsistent_gap == 0.0


def test_replay_negative_value_gap():
    # rint(-2.45) = -2; imposing -3 is inconsistent. frac(-2.45) = 0.55, so
    # the gap is 0.05 (a gap measured to the integer would give 0.45).
    one = np.ones((1, 1))
    rep = O.replay(np.array([[-2.45]]), one, one, (0, 0, 1), O.SCALE_NONE, None,
                   np.array([[-3.0]]))
    assert rep.inconsistent == 1
    assert rep.max_inconsistent_gap == pytest.approx(0.05, abs=1e-14)


def test_replay_propagates_the_imposed_error():
    # 1 x 2, no output side (L^B = 1), L^A[1, 0] = 0.5: the error of entry
    # (0, 0) reaches (0, 1) with weight 0.5 (§3.2, the rank-1 update).
    # Imposing codes (1, 1): entry (0, 0) is rounded at 0.4 (rint gives 0, so
    # it is inconsistent, gap 0.1) with error 1 - 0.4 = 0.6, so entry (0, 1) is
    # rounded at 1.0 + 0.5 * 0.6 = 1.3, whose rint is the imposed 1.
    # A free solve would have carried the error 0 - 0.4 instead: 0.8.
    W = np.array([[0.4, 1.0]])
    LA = np.array([[1.0, 0.0], [0.5, 1.0]])
    LB = np.ones((1, 1))
    rep = O.replay(W, LA, LB, (0, 0, 1), O.SCALE_NONE, None, np.array([[1.0, 1.0]]))
    assert rep.inconsistent == 1
    assert rep.max_inconsistent_gap == pytest.approx(0.1, abs=1e-15)
    np.testing.assert_allclose(rep.Wt, [[0.4, 1.3]], atol=1e-15)
    free = O.solve_naive_py(W, LA, LB, (0, 0, 1))
    np.testing.assert_allclose(free.Wt, [[0.4, 0.8]], atol=1e-15)


def test_replay_uses_scales_for_the_gap():
    # row scale 0.5: the value 1.2 is 2.4 code units; rint gives 2, so the
    # imposed 3 is inconsistent at gap 0.1 in code units.
    one = np.ones((1, 1))
    rep = O.replay(np.array([[1.2]]), one, one, (-8, 7, 0), O.SCALE_ROW, np.array([0.5]),
                   np.array([[3.0]]))
    assert rep.inconsistent == 1
    assert rep.max_inconsistent_gap == pytest.approx(0.1, abs=1e-14)


# ------------------------------------------------------- Corollary 3.4 ----

def test_corollary_3_4_bounds_hand_2x2():
    # RevCholesky: A = R^T R with R lower. For a 2 x 2 [[a, b], [b, c]]:
    # r22 = sqrt(c), r21 = b / sqrt(c), r11^2 = a - b^2 / c, so
    # sum_j r_jj^2 = a - b^2/c + c.
    # A = [[2, 1], [1, 2]]: 2 - 1/2 + 2 = 3.5.  B = [[3, 1], [1, 1]]: 3 - 1 + 1 = 3.
    # middle bound 1/4 * 3 * 3.5 = 2.625; outer 1/4 * tr A * tr B = 1/4 * 4 * 4 = 4.
    A = np.array([[2.0, 1.0], [1.0, 2.0]])
    B = np.array([[3.0, 1.0], [1.0, 1.0]])
    mid, outer = O.corollary_3_4_bounds(A, B)
    assert mid == pytest.approx(2.625, rel=1e-14)
    assert outer == pytest.approx(4.0, rel=1e-15)


def test_corollary_3_4_bounds_diagonal_hessians_coincide():
    # diagonal A, B: R = sqrt(A), so r_jj^2 = A_jj and the middle bound is
    # 1/4 tr(A) tr(B), equal to the outer one: 1/4 * (1 + 2 + 5) * (3 + 4) = 14.
    A = np.diag([1.0, 2.0, 5.0])
    B = np.diag([3.0, 4.0])
    mid, outer = O.corollary_3_4_bounds(A, B)
    assert mid == pytest.approx(14.0, rel=1e-15)
    assert outer == pytest.approx(14.0, rel=1e-15)


def test_corollary_3_4_middle_bound_is_attained_by_midpoint_errors():
    # With diagonal Hessians every entry is rounded on its own (no updates),
    # and an entry at a midpoint has error 1/2, contributing A_jj B_ii / 4:
    # all entries at midpoints give exactly the middle bound.
    A = np.diag([2.0, 3.0])
    B = np.diag([5.0])
    W = np.array([[0.5, 1.5]])
    LA, _ = O.factor(A)
    LB, _ = O.factor(B)
    r = O.solve_naive_py(W, LA, LB, (0, 0, 1))
    mid, _ = O.corollary_3_4_bounds(A, B)
    assert O.loss(W, r.V, A, B) == pytest.approx(mid, rel=1e-14)
    assert mid == pytest.approx(0.25 * 5.0 * (2.0 + 3.0), rel=1e-15)
