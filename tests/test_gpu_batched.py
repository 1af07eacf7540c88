"""Batched solve (bakron_solve_batched): several problems of one shape in the
same launches. Every problem's result must equal the single-problem solve on
the same inputs bit for bit (same kernels, same order of operations), and,
in float64, the oracle's codes exactly."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import random_problem

from parity_util import oracle_solve, prepare, to_dev

pytestmark = pytest.mark.gpu

CASES = [  # (batch, m, n, alphabet, scale rule)
    (3, 50, 70, (-8, 7, 0), "row"),
    (4, 37, 1, (0, 0, 1), None),
    (2, 130, 97, (-4, 3, 0), "col"),
    (5, 17, 33, (-8, 7, 0), "row"),
    (3, 200, 170, (-8, 7, 0), "row"),  # several band products per problem
]


def _batch_inputs(batch, m, n, dtype, alphabet, rule, seed0):
    hi = alphabet[1] if not alphabet[2] else 7
    out = []
    for b in range(batch):
        p = random_problem(m, n, dtype, seed=seed0 + 31 * b, w_std=2.0 if alphabet[2] else 0.02,
                           heavy_tail=bool(b % 2), samples_factor=3)
        out.append(prepare(p.W, p.A, p.B, dtype, alphabet, rule, hi=max(hi, 1)))
    return out


def _stack(inps, attr):
    return torch.stack([to_dev(getattr(x, attr)) for x in inps])


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("batch,m,n,alphabet,rule", CASES)
def test_batched_equals_single(gpu_lib, dtype, batch, m, n, alphabet, rule):
    bk = gpu_lib
    inps = _batch_inputs(batch, m, n, dtype, alphabet, rule, seed0=m * 7 + n)
    W, LA, LB = _stack(inps, "W"), _stack(inps, "LA"), _stack(inps, "LB")
    s = _stack(inps, "s") if rule else None
    mode = inps[0].mode if rule else None
    Vb, Wtb = bk.solve_batched(W, LA, LB, alphabet, s, scale_mode=mode, return_wt=True)
    for b, inp in enumerate(inps):
        V1, Wt1 = bk.solve(W[b], LA[b], LB[b], alphabet, None if s is None else s[b],
                           scale_mode=mode, return_wt=True)
        torch.cuda.synchronize()
        assert torch.equal(Vb[b], V1), (b, "codes differ from the single solve")
        assert torch.equal(Wtb[b], Wt1), (b, "values at rounding differ from the single solve")
        if dtype == "f64":
            ref = oracle_solve(inp, naive=(m * n <= 4096))
            np.testing.assert_array_equal(Vb[b].cpu().numpy(), ref.V.astype(np.int32))


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_batched_shared_factors(gpu_lib, dtype):
    """One L^A and one L^B for the whole batch (stride 0), per-problem W and
    row scales; also checked against the oracle in float64."""
    bk = gpu_lib
    batch, m, n = 4, 70, 90
    base = random_problem(m, n, dtype, seed=11, heavy_tail=True, samples_factor=3)
    inps = []
    for b in range(batch):
        p = random_problem(m, n, dtype, seed=100 + b, samples_factor=3)
        inps.append(prepare(p.W, base.A, base.B, dtype, (-8, 7, 0), "row"))
    W, s = _stack(inps, "W"), _stack(inps, "s")
    LA, LB = to_dev(inps[0].LA), to_dev(inps[0].LB)
    Vb = bk.solve_batched(W, LA, LB, (-8, 7, 0), s)
    for b, inp in enumerate(inps):
        V1 = bk.solve(W[b], LA, LB, (-8, 7, 0), s[b])
        torch.cuda.synchronize()
        assert torch.equal(Vb[b], V1), b
        if dtype == "f64":
            ref = oracle_solve(inp)
            np.testing.assert_array_equal(Vb[b].cpu().numpy(), ref.V.astype(np.int32))


def test_batched_single_problem_and_empty(gpu_lib):
    bk = gpu_lib
    inp = _batch_inputs(1, 40, 60, "f64", (-8, 7, 0), "row", seed0=5)[0]
    W, LA, LB, s = (to_dev(getattr(inp, a))[None] for a in ("W", "LA", "LB", "s"))
    Vb = bk.solve_batched(W, LA, LB, (-8, 7, 0), s)
    ref = oracle_solve(inp, naive=True)
    np.testing.assert_array_equal(Vb[0].cpu().numpy(), ref.V.astype(np.int32))
    e = bk.solve_batched(torch.empty((0, 40, 60), dtype=torch.float64, device="cuda"), LA[0], LB[0],
                         (-8, 7, 0))
    assert e.shape == (0, 40, 60)


# ----------------------------------------------------------- batched factor ---

@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("batch,m,n", [(3, 70, 70), (4, 50, 130), (2, 200, 64), (5, 1, 9),
                                       (3, 257, 257)])
def test_factor_batched_equals_single(gpu_lib, dtype, batch, m, n):
    """Every pair's factors equal bakron_factor's bit for bit (both the
    shared-launch case m == n and the two-set case m != n), and match the
    oracle's factor to the factor parity bound."""
    bk = gpu_lib
    probs = [random_problem(m, n, dtype, seed=97 * b + m + n, heavy_tail=bool(b % 2))
             for b in range(batch)]
    A = torch.stack([to_dev(p.A) for p in probs])
    B = torch.stack([to_dev(p.B) for p in probs])
    LA, LB, dA, dB = bk.factor_batched(A, B)
    for b, p in enumerate(probs):
        la, lb, da, db = bk.factor(A[b], B[b])
        torch.cuda.synchronize()
        for x, y in ((LA[b], la), (LB[b], lb), (dA[b], da), (dB[b], db)):
            assert torch.equal(x, y), b
        ref, _ = O.factor(p.A)
        cond = np.linalg.cond(O.sym_from_lower(p.A))
        eps = 1e-16 if dtype == "f64" else 6e-8
        err = np.max(np.abs(LA[b].cpu().numpy().astype(np.float64) - ref))
        assert err <= 8 * eps + 64 * cond * 1.1e-16 * n, err


def test_factor_batched_reports_failing_pair(gpu_lib):
    bk = gpu_lib
    probs = [random_problem(40, 100, "f64", seed=200 + b) for b in range(4)]
    A = torch.stack([to_dev(p.A) for p in probs])
    B = torch.stack([to_dev(p.B) for p in probs])
    A[2, 30, 30] = -5.0  # pair 2, side A, row 30: reversed pivot 100 - 1 - 30
    with pytest.raises(bk.BakronError) as ei:
        bk.factor_batched(A, B)
    assert ei.value.status == bk.ENOTSPD
    assert tuple(ei.value.bad_pivot) == (2, 0, 69)
    B[1, 5, 5] = -1.0  # an earlier pair fails on side B
    with pytest.raises(bk.BakronError) as ei:
        bk.factor_batched(A, B)
    assert tuple(ei.value.bad_pivot) == (1, 1, 34)


# ------------------------------------------------------------- batched loss ---

@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("batch,m,n,rule", [(3, 50, 70, "row"), (2, 130, 97, "col"),
                                            (4, 33, 200, None), (2, 300, 170, "row")])
def test_loss_batched_matches_single_and_oracle(gpu_lib, dtype, batch, m, n, rule):
    """Every problem's batched loss equals bakron_loss to float64 rounding
    (the batched form reduces per block, the single one per stream-K range)
    and the oracle's loss of the same codes to 1e-10."""
    bk = gpu_lib
    alphabet = (-8, 7, 0) if rule else (0, 0, 1)
    inps = _batch_inputs(batch, m, n, dtype, alphabet, rule, seed0=m + 3 * n)
    W, LA, LB = _stack(inps, "W"), _stack(inps, "LA"), _stack(inps, "LB")
    s = _stack(inps, "s") if rule else None
    mode = inps[0].mode if rule else None
    V = bk.solve_batched(W, LA, LB, alphabet, s, scale_mode=mode)
    probs = [random_problem(m, n, dtype, seed=m + 3 * n + 31 * b, w_std=2.0 if alphabet[2] else 0.02,
                            heavy_tail=bool(b % 2), samples_factor=3) for b in range(batch)]
    A = torch.stack([to_dev(p.A) for p in probs])
    B = torch.stack([to_dev(p.B) for p in probs])
    lb = bk.loss_batched(W, V, A, B, s, scale_mode=mode).cpu().numpy()
    for b, inp in enumerate(inps):
        l1 = bk.loss(W[b], V[b], A[b], B[b], None if s is None else s[b], scale_mode=mode)
        assert abs(lb[b] - l1) <= 1e-12 * abs(l1), (b, lb[b], l1)
        lo = O.loss(inp.W, V[b].cpu().numpy(), probs[b].A, probs[b].B, inp.mode, inp.s)
        assert abs(lb[b] - lo) <= 1e-10 * abs(lo), (b, lb[b], lo)


def test_loss_batched_shared_hessians_and_empty(gpu_lib):
    bk = gpu_lib
    p = random_problem(40, 60, "f64", seed=9, samples_factor=3)
    Ws = torch.stack([to_dev(p.W) * (1 + 0.1 * b) for b in range(3)])
    V = torch.zeros(Ws.shape, dtype=torch.int32, device="cuda")
    A, B = to_dev(p.A), to_dev(p.B)
    lb = bk.loss_batched(Ws, V, A, B).cpu().numpy()
    for b in range(3):
        l1 = bk.loss(Ws[b], V[b], A, B)
        assert abs(lb[b] - l1) <= 1e-12 * abs(l1)
    e = bk.loss_batched(torch.zeros((0, 40, 60), dtype=torch.float64, device="cuda"),
                        torch.zeros((0, 40, 60), dtype=torch.int32, device="cuda"), A, B)
    assert e.shape == (0,)


@pytest.mark.timeout(600)
def test_kv28_fp64_batched_all_bit_exact(gpu_lib):
    """All 28 k/v projections (1024 x 2048) in float64 through ONE batched
    solve, each against the oracle on its own oracle factors: codes bit for
    bit, values at rounding within 1e-10 code units."""
    import oracle as O
    from synth import config5
    probs = [config5(i) for i in range(28)]
    W = np.stack([p.W.astype(np.float64) for p in probs])
    facs = [(O.factor(p.A), O.factor(p.B)) for p in probs]
    LA = np.stack([f[0][0] for f in facs])
    LB = np.stack([f[1][0] for f in facs])
    S = np.stack([O.row_scales(W[i], 7, np.float64) for i in range(28)])
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    V, Wt = gpu_lib.solve_batched(t(W), t(LA), t(LB), (-8, 7, 0), t(S), return_wt=True)
    V, Wt = V.cpu().numpy(), Wt.cpu().numpy()
    for i in range(28):
        ref = O.solve_recursive(W[i], LA[i], LB[i], (-8, 7, 0), O.SCALE_ROW, S[i])
        assert np.array_equal(V[i], ref.V.astype(np.int32)), i
        assert np.max(np.abs(Wt[i] - ref.Wt) / S[i][:, None]) <= 1e-10, i
