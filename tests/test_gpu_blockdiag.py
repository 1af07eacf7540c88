"""Block-diagonal output factor on the GPU (per-head attention Grams
assembled block-diagonally, Appendix D / Table 4 of the BaKron paper):
bakron_factor_blockdiag / bakron_solve_blockdiag / bakron_loss_blockdiag
against the float64 oracle on the assembled dense matrix and against the
GPU's dense path, on ragged head sizes and at the full 4096 x 4096
attention shape with 32 heads of 128."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import block_diag, config3_heads, head_grams, random_problem

from parity_util import (Inputs, assert_factor_close, assert_fp32_validity, cond_estimate,
                         fp32_parity, oracle_branch_spread, oracle_solve, to_dev)

pytestmark = pytest.mark.gpu


def _oracle_blocks(blocks):
    fs = [O.factor(blocks[h]) for h in range(blocks.shape[0])]
    return np.stack([f[0] for f in fs]), np.concatenate([f[1] for f in fs])


@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("heads,b,n", [(1, 40, 33), (5, 48, 333), (7, 17, 64)])
def test_factor_blockdiag_matches_oracle(gpu_lib, dtype, heads, b, n):
    dt = np.float64 if dtype == "f64" else np.float32
    p = random_problem(heads * b, n, dtype, seed=heads * 100 + b, heavy_tail=True)
    blocks = head_grams(50 + heads, heads, b, 3 * b).astype(dt)
    LA, LB, dA, dB = gpu_lib.factor_blockdiag(to_dev(p.A), to_dev(blocks))
    eps = 1e-16 if dtype == "f64" else 6e-8
    RA, rdA = O.factor(p.A)
    assert_factor_close(LA.cpu().numpy(), dA.cpu().numpy(), RA, rdA, cond_estimate(p.A, RA, rdA), eps)
    RB, rdB = _oracle_blocks(blocks)
    LB, dB = LB.cpu().numpy(), dB.cpu().numpy()
    for h in range(heads):
        c = cond_estimate(blocks[h], RB[h], rdB[h * b:(h + 1) * b])
        assert_factor_close(LB[h], dB[h * b:(h + 1) * b], RB[h], rdB[h * b:(h + 1) * b], c, eps)


def test_factor_blockdiag_reports_the_failing_block(gpu_lib):
    p = random_problem(4 * 20, 30, "f64", seed=3)
    blocks = head_grams(60, 4, 20, 60)
    blocks[2, 5, 5] = -3.0
    with pytest.raises(gpu_lib.BakronError) as ei:
        gpu_lib.factor_blockdiag(to_dev(p.A), to_dev(blocks))
    assert ei.value.status == gpu_lib.ENOTSPD
    assert ei.value.bad_pivot[0] == 1 and ei.value.bad_pivot[1] == 2


def _solve_all(bk, W, LA, LBb, al, s):
    """Block solve, and the dense solve on the assembled block-diagonal L^B."""
    LBd = block_diag(LBb)
    Vb, Wtb = bk.solve_blockdiag(to_dev(W), to_dev(LA), to_dev(LBb), al, to_dev(s), return_wt=True)
    Vd, Wtd = bk.solve(to_dev(W), to_dev(LA), to_dev(LBd), al, to_dev(s), return_wt=True)
    torch.cuda.synchronize()
    return Vb.cpu().numpy(), Wtb.cpu().numpy(), Vd.cpu().numpy(), Wtd.cpu().numpy(), LBd


@pytest.mark.parametrize("heads,b,n,rule", [(5, 48, 333, "row"), (3, 100, 70, "col"),
                                            (8, 16, 257, "row")])
def test_solve_blockdiag_fp64_equals_dense_and_oracle(gpu_lib, heads, b, n, rule):
    p = random_problem(heads * b, n, "f64", seed=heads + b + n, w_std=0.02, heavy_tail=True)
    blocks = head_grams(70 + heads, heads, b, 3 * b)
    LA, dA = O.factor(p.A)
    LBb, dB = _oracle_blocks(blocks)
    s = O.row_scales(p.W, 7, np.float64) if rule == "row" else O.row_scales(p.W.T, 7, np.float64)
    mode = O.SCALE_ROW if rule == "row" else O.SCALE_COL
    Vb, Wtb, Vd, Wtd, LBd = _solve_all(gpu_lib, p.W, LA, LBb, (-8, 7, 0), s)
    ref = oracle_solve(Inputs(p.W, LA, LBd, dA, dB, s, mode, (-8, 7, 0)))
    assert np.array_equal(Vb, ref.V.astype(np.int32))
    assert np.array_equal(Vb, Vd)
    S = O.scale_grid(heads * b, n, mode, s)
    assert np.max(np.abs(Wtb - ref.Wt) / S) <= 1e-10


def test_solve_blockdiag_fp32_parity(gpu_lib):
    heads, b, n = 6, 64, 300
    p = random_problem(heads * b, n, "f32", seed=11, w_std=0.02, heavy_tail=True)
    blocks = head_grams(80, heads, b, 3 * b)
    LA, dA = O.factor(p.A)
    LBb, dB = _oracle_blocks(blocks)
    LA32, LBb32 = LA.astype(np.float32), LBb.astype(np.float32)
    s = O.row_scales(p.W, 7, np.float32)
    Vb, Wtb, Vd, Wtd, LBd = _solve_all(gpu_lib, p.W, LA32, LBb32, (-8, 7, 0), s)
    inp = Inputs(p.W, LA32, LBd, dA, dB, s, O.SCALE_ROW, (-8, 7, 0))
    ref = oracle_solve(inp)
    rep = fp32_parity(inp, Vb, Wtb, ref, p.A.astype(np.float64), block_diag(blocks))
    if rep.mismatches:
        rep.branch_spread, rep.branch_detail = oracle_branch_spread(inp, ref, dA, dB)
    print(rep.as_dict())
    assert_fp32_validity(rep)
    assert rep.max_dev <= 1e-4


@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_loss_blockdiag_matches_oracle_and_dense(gpu_lib, dtype):
    heads, b, n = 5, 40, 90
    p = random_problem(heads * b, n, dtype, seed=21, w_std=0.02)
    blocks = head_grams(90, heads, b, 3 * b).astype(p.W.dtype)
    s = O.row_scales(p.W, 7)
    V = np.clip(np.rint(p.W / s[:, None]), -8, 7).astype(np.int32)
    l_blk = gpu_lib.loss_blockdiag(to_dev(p.W), to_dev(V), to_dev(p.A), to_dev(blocks), to_dev(s))
    l_dense = gpu_lib.loss(to_dev(p.W), to_dev(V), to_dev(p.A), to_dev(block_diag(blocks)), to_dev(s))
    l_ref = O.loss(p.W, V, p.A, block_diag(blocks), O.SCALE_ROW, s)
    assert abs(l_blk - l_ref) <= 1e-10 * abs(l_ref)
    assert abs(l_blk - l_dense) <= 1e-12 * abs(l_ref)


@pytest.mark.timeout(600)
def test_attn4096_32_heads_fp64_bit_exact(gpu_lib):
    """4096 x 4096 with 32 heads of 128 (the attention projection shape):
    float64 codes of the block path equal the dense GPU path's and the
    oracle's bit for bit; the GPU block factor matches the oracle's."""
    p, blocks = config3_heads(32)
    W = p.W.astype(np.float64)
    A = p.A.astype(np.float64)
    blocks = blocks.astype(np.float64)
    LAg, LBg, dAg, dBg = gpu_lib.factor_blockdiag(to_dev(A), to_dev(blocks))
    LA, dA = O.factor(A)
    LBb, dB = _oracle_blocks(blocks)
    err = max(float(np.max(np.abs(LAg.cpu().numpy() - LA))),
              float(np.max(np.abs(LBg.cpu().numpy() - LBb))))
    assert err <= 1e-9, err
    s = O.row_scales(W, 7, np.float64)
    Vb, Wtb, Vd, Wtd, LBd = _solve_all(gpu_lib, W, LA, LBb, (-8, 7, 0), s)
    ref = oracle_solve(Inputs(W, LA, LBd, dA, dB, s, O.SCALE_ROW, (-8, 7, 0)))
    mism = int(np.count_nonzero(Vb != ref.V.astype(np.int32)))
    dev = float(np.max(np.abs(Wtb - ref.Wt) / s[:, None]))
    print("32 heads fp64: mismatches vs oracle", mism, "vs dense", int(np.count_nonzero(Vb != Vd)),
          "max dev", dev, "factor err", err)
    assert mism == 0
    assert np.array_equal(Vb, Vd)
    assert dev <= 1e-9
