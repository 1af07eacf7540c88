"""CPU pins of the block-diagonal output factor (the per-head attention
Grams assembled block-diagonally, Appendix D / Table 4 of "BaKron: Efficient
Quantization with Kronecker-Factored Hessians", arXiv 2608.06291): the facts
the GPU's per-head decomposition rests on, checked on the oracle."""
import numpy as np

import oracle as O
from synth import block_diag, head_grams, random_problem


def test_factor_of_block_diagonal_is_block_diagonal():
    """Cholesky((blockdiag B_h)^-1) = blockdiag(Cholesky(B_h^-1)): the
    inverse of a block-diagonal matrix is block-diagonal, and the Cholesky
    factor of a block-diagonal SPD matrix is the block-diagonal of the
    blocks' factors (uniqueness of the factor)."""
    blocks = head_grams(99, 4, 7, 20)
    L, d = O.factor(block_diag(blocks))
    for h in range(4):
        Lh, dh = O.factor(blocks[h])
        np.testing.assert_allclose(L[7 * h:7 * h + 7, 7 * h:7 * h + 7], Lh, atol=1e-12)
        np.testing.assert_allclose(d[7 * h:7 * h + 7], dh, rtol=1e-12)
    mask = block_diag(np.ones((4, 7, 7), dtype=bool))
    assert np.all(np.abs(L[~mask]) <= 1e-14)


def test_solve_with_block_diagonal_output_side_splits_by_head():
    """With a block-diagonal L^B an error reaches only rows of its own block,
    so Algorithm 2 on the whole matrix equals Algorithm 2 on each head's rows
    with that head's factor and the shared L^A: codes and values at rounding
    identical (the cross-block terms are exact zeros the loop skips)."""
    heads, b, n = 3, 5, 9
    p = random_problem(heads * b, n, "f64", seed=4, w_std=2.0)
    blocks = head_grams(98, heads, b, 12)
    LA, _ = O.factor(p.A)
    LBb = [O.factor(blocks[h])[0] for h in range(heads)]
    LB = block_diag(np.stack(LBb))
    full = O.solve_naive(p.W, LA, LB, (0, 0, 1))
    for h in range(heads):
        part = O.solve_naive(p.W[h * b:(h + 1) * b], LA, LBb[h], (0, 0, 1))
        assert np.array_equal(part.V, full.V[h * b:(h + 1) * b])
        assert np.array_equal(part.Wt, full.Wt[h * b:(h + 1) * b])


def test_loss_with_block_diagonal_output_side_is_a_sum_over_heads():
    """tr(B D A D^T) = sum_h tr(B_h D_h A D_h^T) for block-diagonal B."""
    heads, b, n = 3, 4, 6
    p = random_problem(heads * b, n, "f64", seed=5, w_std=2.0)
    blocks = head_grams(97, heads, b, 10)
    V = np.rint(p.W)
    total = O.loss(p.W, V, p.A, block_diag(blocks))
    parts = sum(O.loss(p.W[h * b:(h + 1) * b], V[h * b:(h + 1) * b], p.A, blocks[h])
                for h in range(heads))
    assert abs(total - parts) <= 1e-12 * abs(total)
