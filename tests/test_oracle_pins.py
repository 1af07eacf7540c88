"""Pins of the CPU oracle to facts other than itself.

Each test states what fixes the expected value: a hand-derived example, a
closed form, a textbook routine on the materialised problem, or a theorem of
"BaKron: Efficient Quantization with Kronecker-Factored Hessians"
(arXiv 2608.06291). None of these runs on a GPU.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
from synth import random_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

ALPHABETS = [
    ("int", (0, 0, 1), O.SCALE_NONE),
    ("4bit_row", (-8, 7, 0), O.SCALE_ROW),
    ("3bit_col", (-4, 3, 0), O.SCALE_COL),
]


def _scales(p, mode, hi=7):
    if mode == O.SCALE_ROW:
        return O.row_scales(p.W, hi, np.float64)
    if mode == O.SCALE_COL:
        return O.row_scales(np.asarray(p.W).T, hi, np.float64)
    return None


def _prob(m, n, seed, mode):
    # integer alphabet: spread W over several units; bounded: Gaussian weights
    std = 2.0 if mode == O.SCALE_NONE else 1.0
    return random_problem(m, n, "f64", seed=seed, w_std=std, samples_factor=3)


# ---------------------------------------------------------------- golden ----

@pytest.mark.parametrize("fname", ["hand_2x2_integers.json", "hand_2x2_bounded_rowscales.json"])
def test_golden_hand_examples(fname):
    """Small cases worked by hand from §3.2 Algorithm 2 (derivation in the file)."""
    g = json.load(open(os.path.join(GOLDEN, fname)))
    A, B, W = (np.array(g[k]) for k in ("A", "B", "W"))
    al = (g["alphabet"]["lo"], g["alphabet"]["hi"], int(g["alphabet"]["unbounded"]))
    mode = {"none": O.SCALE_NONE, "row": O.SCALE_ROW, "col": O.SCALE_COL}[g["scale_mode"]]
    s = None if g["scales"] is None else np.array(g["scales"])
    LA, dA = O.factor(A)
    LB, dB = O.factor(B)
    if "LhatA" in g:
        np.testing.assert_allclose(LA, g["LhatA"], atol=1e-15)
        np.testing.assert_allclose(LB, g["LhatB"], atol=1e-15)
        np.testing.assert_allclose(dA ** 2, g["dA_squared"], rtol=1e-14)
        np.testing.assert_allclose(dB ** 2, g["dB_squared"], rtol=1e-14)
    for solver in (O.solve_naive, O.solve_naive_py, O.solve_antidiag, O.solve_bakron,
                   O.solve_recursive):
        r = solver(W, LA, LB, al, mode, s)
        assert r.V.tolist() == g["V"], solver.__name__
        np.testing.assert_allclose(r.Wt, g["Wt"], atol=1e-14)
        np.testing.assert_allclose(r.E, g["E"], atol=1e-14)
    r = O.solve_naive(W, LA, LB, al, mode, s)
    assert O.loss(W, r.V, A, B, mode, s) == pytest.approx(g["loss"], rel=1e-13)
    assert O.loss_from_errors(r.E, dA, dB) == pytest.approx(g["loss"], rel=1e-13)


def test_tie_rule_round_half_even():
    """Reading of Appendix B's unnamed tie rule: exact halves go to the even integer."""
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5])
    assert O.quantize(x, 1.0, (0, 0, 1)).tolist() == [0, 2, 2, -0, -2, -2, 4]
    # bounded alphabet clamps after rounding (closest element of {lo..hi})
    assert O.quantize(np.array([9.4, -9.6, 7.49, -8.5]), 1.0, (-8, 7, 0)).tolist() == [7, -8, 7, -8]


# ------------------------------------------------------ §3.1 identities ----

def test_prop_3_1_vec_kron():
    """Proposition 3.1: (A (x) B) vec(W) = vec(B W A^T), with column-major vec."""
    g = np.random.default_rng(11)
    m, n = 5, 7
    A, B, W = g.standard_normal((n, n)), g.standard_normal((m, m)), g.standard_normal((m, n))
    lhs = np.kron(A, B) @ O.vec(W)
    rhs = O.vec(B @ W @ A.T)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=1e-13)
    # vec is column-major: vec(W)[j*m+i] = W[i,j]
    assert O.vec(W)[3 * m + 2] == W[2, 3]


def test_factor_distributes_over_kron():
    """§3.1: Cholesky distributes over the Kronecker product, so the factor of
    the materialised (A (x) B)^-1 is L^A (x) L^B, and so are the normalised ones."""
    p = random_problem(4, 6, "f64", seed=3)
    LA, dA = O.factor(p.A)
    LB, dB = O.factor(p.B)
    LK, dK = O.factor(np.kron(p.A, p.B))
    np.testing.assert_allclose(LK, np.kron(LA, LB), atol=1e-12)
    np.testing.assert_allclose(dK, np.kron(dA, dB), rtol=1e-12)


def test_factor_properties():
    """Cholesky(A^-1) by definition (§3.1): L L^T A = I, lower, positive diagonal;
    normalised columns have unit diagonal; and diag = 1/diag(RevCholesky(A))
    since Cholesky(A^-1) = RevCholesky(A)^-1."""
    p = random_problem(1, 37, "f64", seed=5, heavy_tail=True)
    L, d = O.factor(p.A)
    Lfull = L * d[None, :]
    np.testing.assert_allclose(Lfull @ Lfull.T @ O.sym_from_lower(p.A), np.eye(37), atol=1e-9)
    assert np.all(np.triu(L, 1) == 0)
    assert np.all(np.diag(L) == 1.0)
    assert np.all(d > 0)
    R = O.rev_cholesky(p.A)
    np.testing.assert_allclose(R.T @ R, O.sym_from_lower(p.A), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d, 1.0 / np.diag(R), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.inv(R) / np.diag(np.linalg.inv(R))[None, :], L, atol=1e-10)


def test_factor_reads_lower_triangle_only():
    p = random_problem(1, 9, "f64", seed=6)
    junk = np.triu(np.full((9, 9), 1e6), 1) + np.tril(p.A)
    np.testing.assert_array_equal(O.factor(junk)[0], O.factor(p.A)[0])


@pytest.mark.parametrize("Ab", [np.array([[1.0, 2.0], [2.0, 1.0]]), -np.eye(3),
                                np.zeros((4, 4)), np.array([[1.0, 1.0], [1.0, 1.0]])])
def test_non_spd_rejected(Ab):
    with pytest.raises(np.linalg.LinAlgError):
        O.factor(Ab)


# ------------------------------------------- brute force on tiny inputs ----

@pytest.mark.parametrize("name,al,mode", ALPHABETS)
@pytest.mark.parametrize("m,n,seed", [(3, 4, 0), (5, 3, 1), (6, 6, 2), (1, 5, 3), (4, 1, 4)])
def test_materialised_hessian_gptq(name, al, mode, m, n, seed):
    """Algorithm 2 is Algorithm 1 on vec(W) with H = A (x) B (§3.2). Run the
    textbook vector GPTQ on the materialised mn x mn Hessian and compare."""
    p = _prob(m, n, seed, mode)
    s = _scales(p, mode)
    LA, _ = O.factor(p.A)
    LB, _ = O.factor(p.B)
    r = O.solve_naive(p.W, LA, LB, al, mode, s)
    svec = O.vec(O.scale_grid(m, n, mode, s))
    codes, wt = O.gptq_vector(O.vec(p.W), np.kron(O.sym_from_lower(p.A), O.sym_from_lower(p.B)),
                              svec, al)
    np.testing.assert_array_equal(O.unvec(codes, m, n), r.V)
    np.testing.assert_allclose(O.unvec(wt, m, n), r.Wt, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("name,al,mode", ALPHABETS[:2])
def test_one_sided_special_cases(name, al, mode):
    """B = I gives row-wise GPTQ with H = A (the GPTQ Hessian X X^T (x) I of
    §1); A = I gives column-wise GPTQ with H = B by the same argument."""
    m, n = 7, 9
    p = _prob(m, n, 21, mode)
    s = _scales(p, mode)
    S = O.scale_grid(m, n, mode, s)
    LA, _ = O.factor(p.A)
    r = O.solve_naive(p.W, LA, np.eye(m), al, mode, s)
    for i in range(m):
        codes, wt = O.gptq_vector(p.W[i], p.A, S[i], al)
        np.testing.assert_array_equal(codes, r.V[i])
        np.testing.assert_allclose(wt, r.Wt[i], rtol=1e-10, atol=1e-10)
    LB, _ = O.factor(p.B)
    r2 = O.solve_naive(p.W, np.eye(n), LB, al, mode, s)
    for j in range(n):
        codes, wt = O.gptq_vector(p.W[:, j], p.B, S[:, j], al)
        np.testing.assert_array_equal(codes, r2.V[:, j])


def test_single_entry_is_rounding():
    """m = n = 1 is the base case of Algorithm 5: V = quantize(W)."""
    for x in (0.3, -2.7, 5.5, 4.5):
        r = O.solve_naive(np.array([[x]]), np.eye(1), np.eye(1), (0, 0, 1))
        assert r.V[0, 0] == np.rint(x)
        r = O.solve_naive(np.array([[x]]), np.eye(1), np.eye(1), (-2, 1, 0), O.SCALE_ROW, [0.5])
        assert r.V[0, 0] == np.clip(np.rint(x / 0.5), -2, 1)


def test_diagonal_hessians_give_rtn():
    """Diagonal A, B have Cholesky(inverse) diagonal, so the normalised factors
    are identities (unit diagonal, Appendix B) and no error propagates:
    the result is round-to-nearest."""
    g = np.random.default_rng(2)
    m, n = 9, 11
    W = 3 * g.standard_normal((m, n))
    A = np.diag(g.uniform(0.5, 3, n))
    B = np.diag(g.uniform(0.5, 3, m))
    LA, _ = O.factor(A)
    LB, _ = O.factor(B)
    assert np.array_equal(LA, np.eye(n)) and np.array_equal(LB, np.eye(m))
    s = O.row_scales(W, 7, np.float64)
    r = O.solve_naive(W, LA, LB, (-8, 7, 0), O.SCALE_ROW, s)
    np.testing.assert_array_equal(r.V, O.quantize(W, s[:, None], (-8, 7, 0)))
    np.testing.assert_array_equal(r.Wt, W)


def test_already_quantised_input_is_fixed_point():
    """If W already lies on the scaled grid, every error is zero: V = W/s, loss 0."""
    p = random_problem(12, 10, "f64", seed=8)
    g = np.random.default_rng(4)
    s = g.uniform(0.1, 1.0, 12)
    codes = g.integers(-8, 8, (12, 10)).astype(np.float64)
    W = s[:, None] * codes
    LA, _ = O.factor(p.A)
    LB, _ = O.factor(p.B)
    r = O.solve_recursive(W, LA, LB, (-8, 7, 0), O.SCALE_ROW, s, leaf=4)
    np.testing.assert_array_equal(r.V, codes)
    assert O.loss(W, r.V, p.A, p.B, O.SCALE_ROW, s) == pytest.approx(0.0, abs=1e-20)


# ----------------------------------------------- Theorem 3.2 and friends ----

SHAPES = [(1, 1), (1, 8), (8, 1), (2, 3), (5, 6), (6, 5), (13, 9), (16, 16), (21, 34)]


@pytest.mark.parametrize("name,al,mode", ALPHABETS)
@pytest.mark.parametrize("m,n", SHAPES)
def test_theorem_3_2_four_algorithms_agree(name, al, mode, m, n):
    """Theorem 3.2: naive (both loop orders, Appendix B), antidiagonal,
    recursive and BaKron give the same codes. Float64, so the pre-rounding
    values agree to rounding error."""
    p = _prob(m, n, m * 100 + n, mode)
    s = _scales(p, mode)
    LA, _ = O.factor(p.A)
    LB, _ = O.factor(p.B)
    ref = O.solve_naive(p.W, LA, LB, al, mode, s)
    others = [O.solve_naive(p.W, LA, LB, al, mode, s, order="row"),
              O.solve_antidiag(p.W, LA, LB, al, mode, s),
              O.solve_bakron(p.W, LA, LB, al, mode, s),
              O.solve_recursive(p.W, LA, LB, al, mode, s, leaf=1),
              O.solve_recursive(p.W, LA, LB, al, mode, s, leaf=4)]
    if m * n <= 200:
        others.append(O.solve_naive_py(p.W, LA, LB, al, mode, s))
    for r in others:
        np.testing.assert_array_equal(r.V, ref.V)
        np.testing.assert_allclose(r.Wt, ref.Wt, rtol=1e-9, atol=1e-9)
        np.testing.assert_allclose(r.E, ref.E, rtol=1e-9, atol=1e-9)


def test_fast_oracle_equals_naive_256():
    """The fast oracle (Algorithm 5, C leaves of 32) equals Algorithm 2 at a
    size spanning many leaves, with the 512x512 workload's input recipe."""
    p = random_problem(256, 192, "f64", seed=77, w_std=0.02, heavy_tail=True)
    s = O.row_scales(p.W, 7, np.float64)
    LA, _ = O.factor(p.A)
    LB, _ = O.factor(p.B)
    a = O.solve_naive(p.W, LA, LB, (-8, 7, 0), O.SCALE_ROW, s)
    b = O.solve_recursive(p.W, LA, LB, (-8, 7, 0), O.SCALE_ROW, s)
    np.testing.assert_array_equal(a.V, b.V)
    np.testing.assert_allclose(a.Wt, b.Wt, rtol=1e-9, atol=1e-12)


def test_loss_identity_from_errors():
    """loss = sum_ij E_ij^2/(dB_i dA_j)^2 (v - w = Lhat e and
    Lhat^T (A (x) B) Lhat = diag(dA (x) dB)^-2, the structure of Theorem 3.3)."""
    for mode_i, (name, al, mode) in enumerate(ALPHABETS):
        p = _prob(17, 23, 90 + mode_i, mode)
        s = _scales(p, mode)
        LA, dA = O.factor(p.A)
        LB, dB = O.factor(p.B)
        r = O.solve_recursive(p.W, LA, LB, al, mode, s, leaf=8)
        direct = O.loss(p.W, r.V, p.A, p.B, mode, s)
        assert O.loss_from_errors(r.E, dA, dB) == pytest.approx(direct, rel=1e-10)
        # the loss is also the brute-force quadratic form with the materialised Hessian
        D = O.vec(p.W - O.scale_grid(17, 23, mode, s) * r.V)
        H = np.kron(O.sym_from_lower(p.A), O.sym_from_lower(p.B))
        assert float(D @ H @ D) == pytest.approx(direct, rel=1e-10)


@pytest.mark.parametrize("seed", range(4))
def test_corollary_3_4_bound(seed):
    """Corollary 3.4 (integer alphabet): loss <= 1/4 sum (R^B_ii R^A_jj)^2 <= 1/4 tr A tr B."""
    p = random_problem(15, 12, "f64", seed=seed, w_std=5.0)
    LA, _ = O.factor(p.A)
    LB, _ = O.factor(p.B)
    r = O.solve_recursive(p.W, LA, LB, (0, 0, 1), leaf=4)
    L = O.loss(p.W, r.V, p.A, p.B)
    mid, outer = O.corollary_3_4_bounds(p.A, p.B)
    assert L <= mid * (1 + 1e-12) and mid <= outer * (1 + 1e-12)


def test_hessian_scale_invariance():
    """Appendix A: the algorithms are invariant under scaling the Hessian.
    Powers of two keep every float exactly proportional, so codes are equal."""
    p = random_problem(14, 11, "f64", seed=31, w_std=1.0)
    s = O.row_scales(p.W, 7, np.float64)
    al = (-8, 7, 0)
    base = O.solve_recursive(p.W, *(O.factor(p.A)[0], O.factor(p.B)[0]), al, O.SCALE_ROW, s, leaf=4)
    scaled = O.solve_recursive(p.W, O.factor(4.0 * p.A)[0], O.factor(0.125 * p.B)[0], al,
                               O.SCALE_ROW, s, leaf=4)
    np.testing.assert_array_equal(base.V, scaled.V)


def test_transpose_symmetry():
    """Swapping the roles of rows and columns (W^T, with A and B exchanged
    and row scales turned into column scales) transposes the result: the
    dependency order i<=p, j<=q is symmetric (Appendix B)."""
    p = random_problem(9, 13, "f64", seed=41, w_std=1.0)
    s = O.row_scales(p.W, 7, np.float64)
    LA, _ = O.factor(p.A)
    LB, _ = O.factor(p.B)
    a = O.solve_recursive(p.W, LA, LB, (-8, 7, 0), O.SCALE_ROW, s, leaf=4)
    b = O.solve_recursive(p.W.T, LB, LA, (-8, 7, 0), O.SCALE_COL, s, leaf=4)
    np.testing.assert_array_equal(a.V, b.V.T)


def test_replay_accepts_own_codes_and_flags_a_flip():
    """Re-running recurrence (2) with the oracle's own codes is consistent;
    flipping one code is detected downstream or at the entry itself."""
    p = random_problem(20, 20, "f64", seed=51, w_std=1.0)
    s = O.row_scales(p.W, 7, np.float64)
    LA, _ = O.factor(p.A)
    LB, _ = O.factor(p.B)
    r = O.solve_recursive(p.W, LA, LB, (-8, 7, 0), O.SCALE_ROW, s, leaf=8)
    rep = O.replay(p.W, LA, LB, (-8, 7, 0), O.SCALE_ROW, s, r.V, leaf=8)
    assert rep.inconsistent == 0
    V2 = r.V.copy()
    V2[3, 4] = V2[3, 4] + (1 if V2[3, 4] < 7 else -1)
    rep2 = O.replay(p.W, LA, LB, (-8, 7, 0), O.SCALE_ROW, s, V2, leaf=8)
    assert rep2.inconsistent >= 1


# ------------------------------------------- planted mistakes are caught ----

def _naive_variant(W, LA, LB, al, mode, s, bug):
    """Pure-Python Algorithm 2 with one plausible mistake planted (CPU only)."""
    W = np.array(W, dtype=np.float64)
    m, n = W.shape
    S = O.scale_grid(m, n, mode, s)
    V = np.zeros((m, n))
    Wt = np.zeros((m, n))
    for j in range(n):
        for i in range(m):
            x = W[i, j]
            c = O.quantize(x, S[i, j], al)
            e = S[i, j] * c - x
            if bug == "sign":
                e = -e
            V[i, j] = c
            Wt[i, j] = x
            a = LA[:, j] if bug != "transpose_A" else LA[j, :]
            b = LB[:, i] if bug != "rows_for_cols" else LB[:, min(j, m - 1)]
            upd = np.outer(b, a) * e
            if bug == "drop_cross_term":
                upd[i + 1:, j + 1:] = 0.0
            W = W + upd
    return V, Wt


@pytest.mark.parametrize("bug", ["sign", "transpose_A", "rows_for_cols", "drop_cross_term"])
def test_pins_catch_planted_mistakes(bug):
    """A mistake planted in an Algorithm 2 loop makes the materialised-Hessian
    brute-force pin (codes equal and pre-rounding values within 1e-9) fail,
    so that pin can tell a wrong oracle from a right one."""
    m, n = 6, 7
    p = random_problem(m, n, "f64", seed=61, w_std=2.0)
    LA, _ = O.factor(p.A)
    LB, _ = O.factor(p.B)
    codes, wt = O.gptq_vector(O.vec(p.W), np.kron(O.sym_from_lower(p.A), O.sym_from_lower(p.B)),
                              1.0, (0, 0, 1))
    codes, wt = O.unvec(codes, m, n), O.unvec(wt, m, n)

    def pin_holds(V, Wt):
        return np.array_equal(V, codes) and np.allclose(Wt, wt, rtol=1e-9, atol=1e-9)

    assert pin_holds(*_naive_variant(p.W, LA, LB, (0, 0, 1), O.SCALE_NONE, None, None))
    assert not pin_holds(*_naive_variant(p.W, LA, LB, (0, 0, 1), O.SCALE_NONE, None, bug))
