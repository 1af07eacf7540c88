"""Pins of the oracle's Kronecker-factor estimation (§4.2 and Appendix A.2 of
the BaKron paper): the K-FAC factors E[aa^T], E[bb^T] and the Shampoo-style
power iteration, against facts fixed independently of their code: a
hand-computed Gram, exactness of K-FAC when one side is constant, the
rearrangement operator of the best-Kronecker-approximation argument built
from its definition, and the SVD of the rearranged Hessian."""
import numpy as np
import pytest

import oracle as O


def test_weighted_gram_by_hand():
    X = np.array([[1.0, 2.0], [3.0, -1.0]])
    w = np.array([2.0, 0.5])
    # (2 * [[1,2],[2,4]] + 0.5 * [[9,-3],[-3,1]]) / 2
    expect = np.array([[2 + 4.5, 4 - 1.5], [4 - 1.5, 8 + 0.5]]) / 2
    np.testing.assert_allclose(O.weighted_gram(X, w), expect, rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.weighted_gram(X), (np.array([[10.0, -1.0], [-1.0, 5.0]])) / 2,
                               rtol=0, atol=1e-15)
    G = O.damp(O.weighted_gram(X), 0.1)
    # mean diagonal (5 + 2.5) / 2 = 3.75, plus 0.375 on the diagonal
    np.testing.assert_allclose(np.diag(G), [5.375, 2.875], rtol=0, atol=1e-15)
    assert O.weighted_gram(np.zeros((0, 3))).shape == (3, 3)


def _hessian(Xa, Xb):
    """H = E[a a^T (x) b b^T], materialised (library Kronecker product)."""
    N = Xa.shape[0]
    return sum(np.kron(np.outer(a, a), np.outer(b, b)) for a, b in zip(Xa, Xb)) / N


def _rearrange(H, n, m):
    """Van Loan's rearrangement: H of (n m) x (n m) with m x m blocks H_ij
    (i, j < n) maps to the n^2 x m^2 matrix whose row (i, j) is vec(H_ij)^T
    (column-major vec), so that R(A (x) B) = vec(A) vec(B)^T."""
    R = np.empty((n * n, m * m))
    for j in range(n):
        for i in range(n):
            R[i + n * j] = H[i * m:(i + 1) * m, j * m:(j + 1) * m].reshape(-1, order="F")
    return R


def test_rearrangement_definition():
    rng = np.random.default_rng(0)
    A, B = rng.standard_normal((3, 3)), rng.standard_normal((2, 2))
    R = _rearrange(np.kron(A, B), 3, 2)
    np.testing.assert_allclose(R, np.outer(A.reshape(-1, order="F"), B.reshape(-1, order="F")),
                               atol=1e-14)


def test_kfac_is_exact_when_one_side_is_constant():
    """With b_k = b for every sample, E[a a^T (x) b b^T] = E[a a^T] (x) b b^T
    exactly: the independence assumption holds."""
    rng = np.random.default_rng(1)
    Xa = rng.standard_normal((7, 3))
    b = rng.standard_normal(2)
    Xb = np.tile(b, (7, 1))
    A, B = O.kfac_factors(Xa, Xb)
    np.testing.assert_allclose(np.kron(A, B), _hessian(Xa, Xb), atol=1e-13)
    np.testing.assert_allclose(B, np.outer(b, b), atol=1e-14)


def test_shampoo_one_step_is_one_power_step_on_the_rearranged_hessian():
    """u = R(H) v, v = R(H)^T u from v = vec(I_m), u = vec(I_n): one step
    gives vec(A1) = R(H) vec(I_m), vec(B1) = R(H)^T vec(I_n)."""
    rng = np.random.default_rng(2)
    n, m, N = 3, 4, 9
    Xa, Xb = rng.standard_normal((N, n)), rng.standard_normal((N, m))
    R = _rearrange(_hessian(Xa, Xb), n, m)
    A1, B1 = O.shampoo_factors(Xa, Xb, iters=1)
    np.testing.assert_allclose(A1.reshape(-1, order="F"), R @ np.eye(m).reshape(-1, order="F"),
                               atol=1e-12)
    np.testing.assert_allclose(B1.reshape(-1, order="F"), R.T @ np.eye(n).reshape(-1, order="F"),
                               atol=1e-12)
    # and equals the closed form of the paper for a single iteration
    np.testing.assert_allclose(A1, O.weighted_gram(Xa, O.sample_sqnorms(Xb)), atol=1e-13)
    np.testing.assert_allclose(B1, O.weighted_gram(Xb, O.sample_sqnorms(Xa)), atol=1e-13)


def test_shampoo_iteration_converges_to_best_kronecker_approximation():
    """Many iterations give the top singular pair of R(H) (numpy SVD), i.e.
    the best Kronecker approximation, which fits H at least as well as
    K-FAC (both scaled optimally)."""
    rng = np.random.default_rng(3)
    n, m, N = 3, 3, 12
    Xa = rng.standard_normal((N, n)) * np.array([3.0, 1.0, 0.3])
    Xb = rng.standard_normal((N, m)) + Xa[:, :m] * 0.8  # correlated sides
    H = _hessian(Xa, Xb)
    R = _rearrange(H, n, m)
    U, S, Vt = np.linalg.svd(R)
    A, B = O.shampoo_factors(Xa, Xb, iters=60)
    a = A.reshape(-1, order="F") / np.linalg.norm(A)
    b = B.reshape(-1, order="F") / np.linalg.norm(B)
    assert abs(abs(a @ U[:, 0]) - 1) < 1e-10
    assert abs(abs(b @ Vt[0]) - 1) < 1e-10

    def fit(A, B):
        K = np.kron(A, B)
        return np.linalg.norm(H - K * (np.sum(H * K) / np.sum(K * K)))

    Ak, Bk = O.kfac_factors(Xa, Xb)
    assert fit(A, B) <= fit(Ak, Bk) + 1e-12
    assert fit(A, B) == pytest.approx(np.sqrt(np.sum(S[1:] ** 2)), rel=1e-9)
