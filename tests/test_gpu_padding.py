"""Ragged shapes and the padding of the last tile row and column.

An error at (i, j) only reaches entries (p, q) with p >= i and q >= j
(§3.3 of the BaKron paper), so the entries that pad an m x n matrix to whole
16 x 16 tiles can never change the real ones, whatever the padding does. The
solve of an m x n problem must therefore equal, bit for bit, the top-left
m x n block of the same problem written out with zero rows and columns of W
(unit rows and columns of the factors, scale 1) up to whole tiles: the tile
grid and every operation on the real entries are the same. Checked with
alphabets that exclude 0, where the padding entries round to a nonzero code
and carry nonzero errors of their own, in both element types, and against
the oracle for the same ragged problems."""
import numpy as np
import pytest
import torch

from synth import random_problem

from parity_util import (assert_fp32_parity, fp32_parity, gpu_solve, oracle_solve, prepare,
                         to_dev)

pytestmark = pytest.mark.gpu

T = 16
# (lo, hi, unbounded), scale rule, largest code for the absmax scale
ALPHAS = [((1, 15, 0), "row", 15), ((-8, -1, 0), "row", 8), ((2, 9, 0), "col", 9),
          ((-8, 7, 0), "row", 7)]
SHAPES = [(1, 1), (17, 33), (50, 70), (130, 97), (33, 200), (211, 45)]


def _pad_to_tiles(inp):
    m, n = inp.W.shape
    mp, np_ = -(-m // T) * T, -(-n // T) * T
    W = np.zeros((mp, np_), inp.W.dtype)
    W[:m, :n] = inp.W
    LA = np.eye(np_, dtype=inp.LA.dtype)
    LA[:n, :n] = inp.LA
    LB = np.eye(mp, dtype=inp.LB.dtype)
    LB[:m, :m] = inp.LB
    s = None
    if inp.s is not None:
        d = mp if inp.mode == 1 else np_
        s = np.ones(d, inp.s.dtype)
        s[:inp.s.shape[0]] = inp.s
    return W, LA, LB, s


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("m,n", SHAPES)
def test_ragged_equals_padded_block(gpu_lib, dtype, m, n):
    bk = gpu_lib
    for k, (al, rule, hi) in enumerate(ALPHAS):
        p = random_problem(m, n, dtype, seed=900 + 7 * m + n + k, w_std=0.02,
                           heavy_tail=bool(k % 2), samples_factor=2)
        inp = prepare(p.W, p.A, p.B, dtype, al, rule, hi=hi)
        V, Wt = gpu_solve(bk, inp)
        Wp, LAp, LBp, sp = _pad_to_tiles(inp)
        Vp, Wtp = bk.solve(to_dev(Wp), to_dev(LAp), to_dev(LBp), al,
                           None if sp is None else to_dev(sp),
                           scale_mode=inp.mode if sp is not None else None, return_wt=True)
        torch.cuda.synchronize()
        Vp, Wtp = Vp.cpu().numpy(), Wtp.cpu().numpy()
        assert np.array_equal(V, Vp[:m, :n]), (m, n, al, rule)
        assert np.array_equal(Wt, Wtp[:m, :n]), (m, n, al, rule)
        # the codes lie in the alphabet, padding included
        assert Vp.min() >= al[0] and Vp.max() <= al[1]


@pytest.mark.parametrize("m,n", [(17, 33), (50, 70), (130, 97)])
def test_zero_free_alphabet_matches_oracle(gpu_lib, m, n):
    """Alphabets without 0: float64 codes identical to the oracle's, float32
    codes within the near-tie bounds of the float32 parity check."""
    for k, (al, rule, hi) in enumerate(ALPHAS[:3]):
        p = random_problem(m, n, "f64", seed=300 + m + k, w_std=0.02, samples_factor=2)
        inp = prepare(p.W, p.A, p.B, "f64", al, rule, hi=hi)
        V, _ = gpu_solve(gpu_lib, inp, return_wt=False)
        ref = oracle_solve(inp)
        assert np.array_equal(V, ref.V.astype(np.int32)), (m, n, al)

        p32 = random_problem(m, n, "f32", seed=300 + m + k, w_std=0.02, samples_factor=2)
        inp32 = prepare(p32.W, p32.A, p32.B, "f32", al, rule, hi=hi)
        V32, Wt32 = gpu_solve(gpu_lib, inp32)
        rep = fp32_parity(inp32, V32, Wt32, oracle_solve(inp32), p32.A, p32.B)
        assert_fp32_parity(rep)
