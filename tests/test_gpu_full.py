"""Full-size parity on the benchmark workloads: the GPU path, in the launch
configuration bench.py times, against the float64 fast oracle (Algorithm 5,
equal to Algorithm 2 by Theorem 3.2 and by the CPU pins) on every output."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import config3

from parity_util import (assert_factor_close, assert_fp32_validity, cond_estimate, fp32_parity,
                         gpu_solve, oracle_branch_spread, oracle_solve, prepare, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cfg3():
    p = config3()
    inp = prepare(p.W, p.A, p.B, "f32", (-8, 7, 0), "row", 7)
    return p, inp


@pytest.mark.timeout(600)
def test_attn4096_factor_matches_oracle(gpu_lib, cfg3):
    p, inp = cfg3
    LA, LB, dA, dB = gpu_lib.factor(to_dev(p.A), to_dev(p.B))
    LA = LA.cpu().numpy().astype(np.float64)
    LB = LB.cpu().numpy().astype(np.float64)
    # oracle factors rounded once to float32; the GPU rounds its float64 result once
    assert np.max(np.abs(LA - inp.LA)) <= 1e-4
    assert np.max(np.abs(LB - inp.LB)) <= 1e-4
    assert np.mean(LA == inp.LA.astype(np.float64)) > 0.5
    np.testing.assert_allclose(dA.cpu().numpy(), inp.dA, rtol=1e-4)
    np.testing.assert_allclose(dB.cpu().numpy(), inp.dB, rtol=1e-4)


@pytest.mark.timeout(600)
def test_attn4096_solve_parity(gpu_lib, cfg3, progress):
    """Float32 at 4096 x 4096 (the parity criteria of the hot path's
    float32 mode, replay and loss parts): every GPU decision the float64
    replay disagrees with is a near-tie within the measured float32
    deviation; the loss differs from the oracle's by at most the oracle's
    own branch spread (measured here) times SPREAD_MULTIPLE, or 1e-4."""
    p, inp = cfg3
    # row scales: the GPU helper equals the oracle's rule bit for bit
    s_gpu = gpu_lib.row_scales(to_dev(inp.W), 7).cpu().numpy()
    np.testing.assert_array_equal(s_gpu, inp.s)
    V, Wt = gpu_solve(gpu_lib, inp)
    ref = oracle_solve(inp)
    progress("4096x4096: float64 oracle solve done")
    rep = fp32_parity(inp, V, Wt, ref, p.A, p.B)
    if rep.mismatches:
        rep.branch_spread, rep.branch_detail = oracle_branch_spread(inp, ref, inp.dA, inp.dB,
                                                                    say=progress)
    print(rep.as_dict(), rep.branch_detail)
    # A float32 solve differs from the float64 one by ~1e-5 code units, so
    # among 16.7M decisions some near-ties flip and each flip cascades into its
    # downstream quadrant: raw agreement is reported, validity is asserted.
    assert_fp32_validity(rep)
    assert rep.max_dev <= 1e-4, rep
    # the GPU loss of the GPU codes equals the oracle's loss of the same codes
    l_gpu = gpu_lib.loss(to_dev(inp.W), to_dev(V), to_dev(p.A), to_dev(p.B), to_dev(inp.s))
    l_ora = O.loss(inp.W, V, p.A, p.B, O.SCALE_ROW, inp.s)
    assert abs(l_gpu - l_ora) <= 1e-9 * abs(l_ora)


@pytest.mark.timeout(600)
def test_attn4096_factor_fp64_matches_oracle(gpu_lib, cfg3):
    """The float64 factor at order 4096 (the workload's A with its 41 outlier
    channels, and B) against the oracle's inverse-then-Cholesky, within the
    condition-scaled bound."""
    p, _ = cfg3
    A64, B64 = p.A.astype(np.float64), p.B.astype(np.float64)
    LA, LB, dA, dB = gpu_lib.factor(to_dev(A64), to_dev(B64))
    for M, L, d in ((A64, LA, dA), (B64, LB, dB)):
        R, rd = O.factor(M)
        c = cond_estimate(M, R, rd)
        err, tol = assert_factor_close(L.cpu().numpy(), d.cpu().numpy(), R, rd, c, 1e-16)
        print("order 4096 fp64 factor: cond <=", c, "max err", err, "tol", tol)


@pytest.mark.timeout(600)
def test_attn4096_fp64_bit_exact(gpu_lib, cfg3):
    """Float64 mode at the full benchmark size: codes identical to the oracle."""
    p, _ = cfg3
    inp = prepare(p.W.astype(np.float64), p.A, p.B, "f64", (-8, 7, 0), "row", 7)
    V, Wt = gpu_solve(gpu_lib, inp)
    ref = oracle_solve(inp)
    mism = int(np.count_nonzero(V != ref.V.astype(np.int32)))
    print("fp64 4096 mismatches", mism, "max dev", float(np.max(np.abs(Wt - ref.Wt) / inp.s[:, None])))
    assert mism == 0
    assert np.max(np.abs(Wt - ref.Wt) / inp.s[:, None]) <= 1e-9


@pytest.mark.timeout(600)
@pytest.mark.parametrize("m,n,alpha,rule", [
    (1509, 2291, (-8, 7, 0), "row"),   # ragged in both directions, 64x64 band tiles on the wide nodes
    (2301, 777, (-4, 3, 0), "col"),    # taller than wide, column scales
    (1111, 1111, (0, 0, 1), None),     # square, integer alphabet, no scales
])
def test_ragged_midsize_fp64_bit_exact(gpu_lib, m, n, alpha, rule):
    """Float64 mode at sizes with many leaf blocks, both band-tile sizes and
    ragged edges in both directions: codes identical to the oracle (its fast
    form, Algorithm 5, pinned to Algorithm 2 on the CPU)."""
    from synth import random_problem
    p = random_problem(m, n, "f64", seed=m * 31 + n, w_std=2.0 if alpha[2] else 0.02,
                       heavy_tail=True, samples_factor=2)
    inp = prepare(p.W, p.A, p.B, "f64", alpha, rule, hi=alpha[1] if not alpha[2] else 7)
    V, Wt = gpu_solve(gpu_lib, inp)
    ref = oracle_solve(inp)
    mism = int(np.count_nonzero(V != ref.V.astype(np.int32)))
    S = O.scale_grid(m, n, inp.mode, inp.s)
    dev = float(np.max(np.abs(Wt - ref.Wt) / S))
    print(m, n, alpha, rule, "mismatches", mism, "max dev", dev)
    assert mism == 0
    assert dev <= 1e-9
