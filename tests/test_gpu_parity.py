"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, on
seeded inputs at sizes the oracle finishes in seconds (several tiles plus
ragged tails), both dtypes, all scale modes, and the edge cases."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import config1, config2, random_problem

from parity_util import (assert_fp32_parity, fp32_parity, gpu_solve, oracle_solve, prepare, tdt,
                         to_dev)

pytestmark = pytest.mark.gpu

ALPHAS = {
    "int": ((0, 0, 1), None),
    "4bit_row": ((-8, 7, 0), "row"),
    "3bit_col": ((-4, 3, 0), "col"),
}
SHAPES = [(1, 1), (1, 37), (37, 1), (16, 16), (17, 33), (50, 70), (100, 64), (130, 97)]


def _problem(m, n, dtype, seed, alpha):
    std = 2.0 if alpha == "int" else 0.02
    return random_problem(m, n, dtype, seed=seed, w_std=std, heavy_tail=(seed % 2 == 1),
                          samples_factor=3)


# ------------------------------------------------------------------ factor ---

# Orders up to 128 run as one fused node (two leaves of 64 and n - 64): 127
# and 128 give second leaves of 63 and 64 rows, 100 one of 36, 192 a node of
# 128 next to a leaf of 64.
@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("m,n", [(1, 1), (5, 9), (16, 16), (64, 64), (65, 130), (127, 128),
                                 (100, 192), (200, 257)])
def test_factor_matches_oracle(gpu_lib, dtype, m, n):
    bk = gpu_lib
    p = random_problem(m, n, dtype, seed=m + n, heavy_tail=True)
    LA, LB, dA, dB = bk.factor(to_dev(p.A), to_dev(p.B))
    LA, LB, dA, dB = (x.cpu().numpy().astype(np.float64) for x in (LA, LB, dA, dB))
    rA, rdA = O.factor(p.A)
    rB, rdB = O.factor(p.B)
    condA = np.linalg.cond(O.sym_from_lower(p.A))
    condB = np.linalg.cond(O.sym_from_lower(p.B))
    eps = 1e-16 if dtype == "f64" else 6e-8
    for L, R, c in ((LA, rA, condA), (LB, rB, condB)):
        assert np.all(np.diag(L) == 1.0)
        assert np.all(np.triu(L, 1) == 0.0)
        tol = 8 * eps + 64 * c * 1.1e-16 * max(L.shape[0], 1)
        assert np.max(np.abs(L - R)) <= tol, (np.max(np.abs(L - R)), tol)
    np.testing.assert_allclose(dA, rdA, rtol=64 * condA * 1.1e-16 * n + 4 * eps)
    np.testing.assert_allclose(dB, rdB, rtol=64 * condB * 1.1e-16 * m + 4 * eps)


# (40, 30): the bad pivot in a single leaf; (100, 110): in the second leaf of
# a fused node (the factor runs on the reversed matrix, so entry 7 is pivot
# n - 8 >= 64)
@pytest.mark.parametrize("m,n", [(40, 30), (100, 110)])
@pytest.mark.parametrize("side", ["A", "B"])
def test_factor_rejects_non_spd(gpu_lib, side, m, n):
    bk = gpu_lib
    p = random_problem(m, n, "f64", seed=1)
    A, B = p.A.copy(), p.B.copy()
    bad = A if side == "A" else B
    bad[7, 7] = -5.0  # indefinite
    with pytest.raises(np.linalg.LinAlgError):
        O.factor(bad)
    with pytest.raises(bk.BakronError) as ei:
        bk.factor(to_dev(A), to_dev(B))
    assert ei.value.status == bk.ENOTSPD
    assert ei.value.bad_pivot[0] == (0 if side == "A" else 1)


@pytest.mark.parametrize("n,i", [(100, 80), (100, 20), (128, 0), (250, 3), (250, 120)])
def test_factor_reports_first_failing_pivot(gpu_lib, n, i):
    """A negative diagonal entry at i of an otherwise SPD matrix: every
    leading principal block of the reversed matrix J A J that excludes i is
    SPD, and the Schur complement at i is A_ii minus a non-negative number,
    so the reversed Cholesky fails first at pivot n-1-i (covers the fused
    order-128 nodes and the levels above them)."""
    bk = gpu_lib
    p = random_problem(30, n, "f64", seed=n + i)
    A = p.A.copy()
    A[i, i] = -5.0
    with pytest.raises(bk.BakronError) as ei:
        bk.factor(to_dev(A), to_dev(p.B))
    assert ei.value.status == bk.ENOTSPD
    assert tuple(ei.value.bad_pivot) == (0, n - 1 - i)


# ------------------------------------------------------------------- solve ---

def test_config1_fp64_bit_exact(gpu_lib):
    """64x64 float64, integer alphabet: codes identical to Algorithm 2."""
    p = config1()
    inp = prepare(p.W, p.A, p.B, "f64", (0, 0, 1))
    V, Wt = gpu_solve(gpu_lib, inp)
    ref = oracle_solve(inp, naive=True)
    np.testing.assert_array_equal(V, ref.V.astype(np.int32))
    np.testing.assert_allclose(Wt, ref.Wt, rtol=1e-10, atol=1e-10)
    l_gpu = gpu_lib.loss(to_dev(p.W), to_dev(V), to_dev(p.A), to_dev(p.B))
    l_ref = O.loss(p.W, ref.V, p.A, p.B)
    assert abs(l_gpu - l_ref) <= 1e-10 * abs(l_ref)


@pytest.mark.parametrize("alpha", list(ALPHAS))
@pytest.mark.parametrize("m,n", SHAPES)
def test_solve_fp64_bit_exact(gpu_lib, m, n, alpha):
    al, rule = ALPHAS[alpha]
    p = _problem(m, n, "f64", 7 * m + n, alpha)
    inp = prepare(p.W, p.A, p.B, "f64", al, rule, hi=7 if alpha != "3bit_col" else 3)
    V, Wt = gpu_solve(gpu_lib, inp)
    ref = oracle_solve(inp, naive=(m * n <= 4096))
    np.testing.assert_array_equal(V, ref.V.astype(np.int32))
    S = O.scale_grid(m, n, inp.mode, inp.s)
    assert np.max(np.abs(Wt - ref.Wt) / S) <= 1e-9


@pytest.mark.parametrize("alpha", list(ALPHAS))
@pytest.mark.parametrize("m,n", SHAPES)
def test_solve_fp32_parity(gpu_lib, m, n, alpha):
    al, rule = ALPHAS[alpha]
    p = _problem(m, n, "f32", 11 * m + n, alpha)
    inp = prepare(p.W, p.A, p.B, "f32", al, rule, hi=7 if alpha != "3bit_col" else 3)
    V, Wt = gpu_solve(gpu_lib, inp)
    ref = oracle_solve(inp)
    rep = fp32_parity(inp, V, Wt, ref, p.A, p.B)
    assert_fp32_parity(rep)
    assert rep.max_dev <= 1e-3, rep


def _strided(x: np.ndarray, ld: int, col0: int) -> torch.Tensor:
    """x as the columns col0 .. col0 + cols - 1 of a wider device buffer whose
    rows are ld elements apart (a leading dimension larger than the row and,
    for odd col0, a start that is not 16-byte aligned)."""
    rows, cols = x.shape
    buf = np.full((rows, ld), np.nan, dtype=x.dtype)
    buf[:, col0:col0 + cols] = x
    return torch.from_numpy(buf).cuda()[:, col0:col0 + cols]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("alpha", ["4bit_row", "3bit_col"])
@pytest.mark.parametrize("ld_pad,col0", [(4, 0), (4, 1), (3, 0), (2, 2)])
def test_strided_operands_equal_contiguous(gpu_lib, dtype, alpha, ld_pad, col0):
    """W, L^A and L^B passed as slices of wider buffers (leading dimension
    larger than the row, aligned or not, rows starting at a misaligned
    address) give the same codes and values bit for bit as contiguous
    operands: the operand packing reads whole 16-byte vectors only where
    every row start allows it and single elements elsewhere, with the same
    per-entry arithmetic; NaN in the unused columns must not leak in."""
    # ragged tile edges on both sides; the contiguous rows (68 and 92 elements)
    # allow 16-byte loads, as do the strided ones with ld_pad 4 (and 2 + 2 in
    # float64); the others start misaligned or have an odd leading dimension
    m, n = 68, 92
    al, rule = ALPHAS[alpha]
    p = _problem(m, n, dtype, 3 * ld_pad + col0, alpha)
    inp = prepare(p.W, p.A, p.B, dtype, al, rule, hi=7 if alpha != "3bit_col" else 3)
    s = to_dev(inp.s)
    V0, Wt0 = gpu_lib.solve(to_dev(inp.W), to_dev(inp.LA), to_dev(inp.LB), inp.alphabet, s,
                            scale_mode=inp.mode, return_wt=True)
    Ws = _strided(inp.W, n + col0 + ld_pad, col0)
    LAs = _strided(inp.LA, n + col0 + ld_pad, col0)
    LBs = _strided(inp.LB, m + col0 + ld_pad, col0)
    V1, Wt1 = gpu_lib.solve(Ws, LAs, LBs, inp.alphabet, s, scale_mode=inp.mode, return_wt=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(V1.cpu().numpy(), V0.cpu().numpy())
    np.testing.assert_array_equal(Wt1.cpu().numpy(), Wt0.cpu().numpy())


def test_config2_fp32_512(gpu_lib):
    """512x512 float32, heavy-tailed input Gram, 4-bit per-row scales."""
    p = config2()
    inp = prepare(p.W, p.A, p.B, "f32", (-8, 7, 0), "row", 7)
    V, Wt = gpu_solve(gpu_lib, inp)
    ref = oracle_solve(inp)
    rep = fp32_parity(inp, V, Wt, ref, p.A, p.B)
    print(rep)
    assert_fp32_parity(rep)


def test_fp64_larger_spanning_band_products(gpu_lib):
    """Large enough (tile anti-diagonals > small-node threshold many times
    over) that the MFMA band products run at several recursion levels."""
    p = random_problem(300, 260, "f64", seed=5, w_std=0.02, heavy_tail=True)
    inp = prepare(p.W, p.A, p.B, "f64", (-8, 7, 0), "row", 7)
    V, Wt = gpu_solve(gpu_lib, inp)
    ref = oracle_solve(inp)
    np.testing.assert_array_equal(V, ref.V.astype(np.int32))
    assert np.max(np.abs(Wt - ref.Wt) / inp.s[:, None]) <= 1e-9


def test_one_sided_B_identity_is_rowwise_gptq(gpu_lib):
    """B = I: the GPU solve equals Algorithm 1 (GPTQ) per row with H = A."""
    p = random_problem(40, 90, "f64", seed=17, w_std=0.02)
    B = np.eye(40)
    inp = prepare(p.W, p.A, B, "f64", (-8, 7, 0), "row", 7)
    V, _ = gpu_solve(gpu_lib, inp)
    for i in range(40):
        codes, _ = O.gptq_vector(p.W[i], p.A, inp.s[i], (-8, 7, 0))
        np.testing.assert_array_equal(V[i], codes.astype(np.int32))


def test_transposed_call_matches(gpu_lib):
    """A column-major caller passes (n, m, W^T, B, A) with column scales; the
    codes are the transpose (the dependency order is symmetric)."""
    p = random_problem(48, 80, "f64", seed=23, w_std=0.02)
    inp = prepare(p.W, p.A, p.B, "f64", (-8, 7, 0), "row", 7)
    V, _ = gpu_solve(gpu_lib, inp)
    inpT = prepare(p.W.T.copy(), p.B, p.A, "f64", (-8, 7, 0), "col", 7)
    VT, _ = gpu_solve(gpu_lib, inpT)
    np.testing.assert_array_equal(V, VT.T)


def test_already_quantised_is_fixed_point(gpu_lib):
    g = np.random.default_rng(3)
    p = random_problem(70, 45, "f32", seed=4)
    s = g.uniform(0.01, 0.1, 70).astype(np.float32)
    codes = g.integers(-8, 8, (70, 45))
    W = (s[:, None].astype(np.float64) * codes).astype(np.float32)
    inp = prepare(W, p.A, p.B, "f32", (-8, 7, 0))
    inp.s, inp.mode = s, O.SCALE_ROW
    V, _ = gpu_solve(gpu_lib, inp)
    np.testing.assert_array_equal(V, codes.astype(np.int32))


# -------------------------------------------------------------- loss, scales --

@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("m,n,mode", [(1, 1, "row"), (37, 50, "row"), (64, 33, "col"),
                                      (130, 97, None), (300, 170, None), (700, 1000, "row")])
def test_loss_matches_oracle(gpu_lib, dtype, m, n, mode):
    p = random_problem(m, n, dtype, seed=m * n, w_std=0.3)
    g = np.random.default_rng(m + n)
    V = g.integers(-8, 8, (m, n)).astype(np.int32)
    s = None
    if mode == "row":
        s = g.uniform(0.01, 0.1, m).astype(p.np_dtype)
    elif mode == "col":
        s = g.uniform(0.01, 0.1, n).astype(p.np_dtype)
    smode = {None: O.SCALE_NONE, "row": O.SCALE_ROW, "col": O.SCALE_COL}[mode]
    ref = O.loss(p.W, V, p.A, p.B, smode, s)
    got = gpu_lib.loss(to_dev(p.W), to_dev(V), to_dev(p.A), to_dev(p.B),
                       None if s is None else to_dev(s), scale_mode=smode if s is not None else None)
    assert abs(got - ref) <= 1e-10 * abs(ref)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_row_scales_bit_exact(gpu_lib, dtype):
    p = random_problem(77, 131, dtype, seed=2, w_std=0.02)
    W = p.W.copy()
    W[5, :] = 0
    for hi in (7, 3):
        got = gpu_lib.row_scales(to_dev(W), hi).cpu().numpy()
        np.testing.assert_array_equal(got, O.row_scales(W, hi))


# ------------------------------------------------------ determinism, streams --

def test_deterministic_reruns(gpu_lib):
    p = random_problem(200, 180, "f32", seed=9, w_std=0.02)
    inp = prepare(p.W, p.A, p.B, "f32", (-8, 7, 0), "row", 7)
    V1, Wt1 = gpu_solve(gpu_lib, inp)
    V2, Wt2 = gpu_solve(gpu_lib, inp)
    np.testing.assert_array_equal(V1, V2)
    np.testing.assert_array_equal(Wt1, Wt2)


def test_concurrent_streams_equal_sequential(gpu_lib):
    bk = gpu_lib
    probs = [random_problem(96, 160, "f32", seed=30 + i, w_std=0.02) for i in range(6)]
    inps = [prepare(p.W, p.A, p.B, "f32", (-8, 7, 0), "row", 7) for p in probs]
    seq = [gpu_solve(bk, inp, return_wt=False)[0] for inp in inps]
    streams = [torch.cuda.Stream() for _ in range(3)]
    dev_in = [(to_dev(i.W), to_dev(i.LA), to_dev(i.LB), to_dev(i.s)) for i in inps]
    torch.cuda.synchronize()
    outs = []
    for k, (W, LA, LB, s) in enumerate(dev_in):
        with torch.cuda.stream(streams[k % 3]):
            outs.append(bk.solve(W, LA, LB, (-8, 7, 0), s))
    torch.cuda.synchronize()
    for a, b in zip(seq, outs):
        np.testing.assert_array_equal(a, b.cpu().numpy())


def test_empty_shapes(gpu_lib):
    bk = gpu_lib
    W = torch.zeros((0, 5), dtype=torch.float32, device="cuda")
    V = bk.solve(W, torch.eye(5, device="cuda"), torch.zeros((0, 0), device="cuda"), (-8, 7, 0))
    assert V.shape == (0, 5)


def test_fp64_bit_exact_random_shapes(gpu_lib):
    """A seeded sweep over 40 random shapes (1..420 rows and columns, so
    every ragged-tail residue mod 16 and up to several leaf blocks and band
    nodes occur), alphabets and scale modes: float64 codes identical to the
    oracle's on every one."""
    rng = np.random.default_rng(2024)
    alphas = [((0, 0, 1), None, 7), ((-8, 7, 0), "row", 7), ((-4, 3, 0), "col", 3),
              ((-3, 3, 0), "row", 3), ((0, 15, 0), "col", 15)]
    for case in range(40):
        m, n = (int(x) for x in rng.integers(1, 421, size=2))
        al, rule, hi = alphas[case % len(alphas)]
        p = random_problem(m, n, "f64", seed=5000 + case, w_std=2.0 if al[2] else 0.02,
                           heavy_tail=bool(case % 2), samples_factor=2)
        inp = prepare(p.W, p.A, p.B, "f64", al, rule, hi=hi)
        V, _ = gpu_solve(gpu_lib, inp, return_wt=False)
        ref = oracle_solve(inp, naive=(m * n <= 2000))
        assert np.array_equal(V, ref.V.astype(np.int32)), (case, m, n, al, rule)


def test_timed_solve_equals_solve_and_times_every_launch(gpu_lib):
    """bakron_solve_timed: the same codes as bakron_solve, and a non-negative
    kernel time for every record of the schedule (leaves and band products)."""
    import ctypes
    bk = gpu_lib
    p = random_problem(700, 500, "f32", seed=9, w_std=0.02, heavy_tail=True, samples_factor=2)
    inp = prepare(p.W, p.A, p.B, "f32", (-8, 7, 0), "row", 7)
    W, LA, LB, s = to_dev(inp.W), to_dev(inp.LA), to_dev(inp.LB), to_dev(inp.s)
    V0 = bk.solve(W, LA, LB, (-8, 7, 0), s)
    ops = bk.solve_schedule(bk.F32, 700, 500)
    op_ms = (ctypes.c_double * len(ops))(*([-5.0] * len(ops)))
    V1 = bk.solve(W, LA, LB, (-8, 7, 0), s, op_ms=op_ms)
    torch.cuda.synchronize()
    assert torch.equal(V0, V1)
    t = list(op_ms)
    assert all(x >= 0.0 for x in t), t
    assert sum(x > 0.0 for x in t) >= len([o for o in ops if o[0] == 0])  # every leaf has work
    assert sum(t) < 1000.0


def test_solve_replays_bit_identically_from_a_captured_graph(gpu_lib):
    """The solve enqueues only kernels on the caller's stream (no host
    synchronisation, no memset, no allocation with a workspace given), so it
    can be captured in a HIP graph: every replay, with eager work and
    synchronisations in between, equals the eager result bit for bit."""
    bk = gpu_lib
    p = random_problem(333, 250, "f32", seed=12, w_std=0.02, heavy_tail=True, samples_factor=2)
    inp = prepare(p.W, p.A, p.B, "f32", (-8, 7, 0), "row", 7)
    W, LA, LB, s = to_dev(inp.W), to_dev(inp.LA), to_dev(inp.LB), to_dev(inp.s)
    ws = torch.empty(bk.workspace_bytes("solve", bk.F32, 333, 250), dtype=torch.uint8, device="cuda")
    V = torch.empty((333, 250), dtype=torch.int32, device="cuda")
    ref = bk.solve(W, LA, LB, (-8, 7, 0), s).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        bk.solve(W, LA, LB, (-8, 7, 0), s, workspace=ws, out=V)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bk.solve(W, LA, LB, (-8, 7, 0), s, workspace=ws, out=V)
    for r in range(3):
        V.fill_(-99)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(V, ref), r
        # eager work between the replays
        other = bk.solve(W, LA, LB, (-8, 7, 0), s)
        torch.cuda.synchronize()
        assert torch.equal(other, ref)
    del g


def test_leaf_wait_give_up_is_reported_and_recoverable(gpu_lib):
    """The leaf blocks' waits for the rows above are bounded. With the bound
    forced to zero from the host (every wait that finds its data not yet
    written gives up at once; every kernel still runs to its end), the solve
    reports BAKRON_EWAIT through bakron_solve_status; with the default bound
    restored, the same workspace gives the normal result and status OK."""
    bk = gpu_lib
    p = random_problem(1024, 768, "f32", seed=21, w_std=0.02, heavy_tail=True, samples_factor=2)
    inp = prepare(p.W, p.A, p.B, "f32", (-8, 7, 0), "row", 7)
    W, LA, LB, s = to_dev(inp.W), to_dev(inp.LA), to_dev(inp.LB), to_dev(inp.s)
    ws = torch.empty(bk.workspace_bytes("solve", bk.F32, 1024, 768), dtype=torch.uint8,
                     device="cuda")
    ref = bk.solve(W, LA, LB, (-8, 7, 0), s, workspace=ws, check=True).clone()
    prev = bk.debug_set_wait_polls(0)
    try:
        with pytest.raises(bk.BakronError) as ei:
            bk.solve(W, LA, LB, (-8, 7, 0), s, workspace=ws, check=True)
        assert ei.value.status == bk.EWAIT
    finally:
        bk.debug_set_wait_polls(prev)
    V = bk.solve(W, LA, LB, (-8, 7, 0), s, workspace=ws, check=True)
    assert torch.equal(V, ref)
