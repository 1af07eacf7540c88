"""bakron_solve_noalloc (the solve with the library's per-GPU scratch, for
callers that cannot allocate) against bakron_solve with a workspace, through
the C ABI: codes and values at rounding bit-identical (same kernels, same
order of operations), on calls in a row whose sizes shrink, in both dtypes,
up to the largest float32 square the scratch holds."""
import numpy as np
import pytest
import torch

from synth import random_problem

pytestmark = pytest.mark.gpu


def _inputs(m, n, dtype, seed, rule):
    p = random_problem(m, n, dtype, seed=seed, w_std=0.02, heavy_tail=True, samples_factor=2)
    tdt = torch.float32 if dtype == "f32" else torch.float64
    dev = "cuda"
    W = torch.from_numpy(p.W).to(dev)
    # unit lower triangular factors with small off-diagonal entries (any such
    # factor is a valid solver input; no factorisation needed here)
    g = torch.Generator(device="cpu").manual_seed(seed)
    LA = (torch.eye(n, dtype=torch.float64) + torch.tril(0.02 * torch.randn(n, n, generator=g, dtype=torch.float64), -1)).to(dev, tdt)
    LB = (torch.eye(m, dtype=torch.float64) + torch.tril(0.02 * torch.randn(m, m, generator=g, dtype=torch.float64), -1)).to(dev, tdt)
    if rule == "row":
        s = W.abs().amax(dim=1) / 7
    elif rule == "col":
        s = W.abs().amax(dim=0) / 7
    else:
        s = None
    return W, LA, LB, (None if s is None else s.contiguous())


def _compare(bk, m, n, dtype, seed, rule, alphabet=(-8, 7, 0)):
    W, LA, LB, s = _inputs(m, n, dtype, seed, rule)
    V_ref, Wt_ref = bk.solve(W, LA, LB, alphabet, s, return_wt=True)
    V = torch.full((m, n), -12345, dtype=torch.int32, device="cuda")
    Wt = torch.full((m, n), float("nan"), dtype=W.dtype, device="cuda")
    out = bk.solve_noalloc(W, LA, LB, alphabet, s, V, Wt)
    torch.cuda.synchronize()
    assert out is V
    assert torch.equal(V, V_ref), (m, n, dtype, rule)
    assert torch.equal(Wt, Wt_ref), (m, n, dtype, rule)
    # a second call without Wt into the same output
    V.fill_(-1)
    bk.solve_noalloc(W, LA, LB, alphabet, s, V)
    torch.cuda.synchronize()
    assert torch.equal(V, V_ref)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_noalloc_matches_solve_on_shrinking_calls(gpu_lib, dtype):
    # first call larger, second smaller (the scratch keeps the first call's
    # contents), third ragged with column scales, fourth unbounded
    _compare(gpu_lib, 700, 900, dtype, 1, "row")
    _compare(gpu_lib, 131, 77, dtype, 2, "row")
    _compare(gpu_lib, 45, 300, dtype, 3, "col")
    _compare(gpu_lib, 64, 64, dtype, 4, None, alphabet=(0, 0, 1))


def test_noalloc_largest_float32_square(gpu_lib):
    # 2496 x 2496 is the largest float32 square whose workspace fits
    assert gpu_lib.workspace_bytes("solve", gpu_lib.F32, 2496, 2496) <= gpu_lib.NOALLOC_SCRATCH_BYTES
    assert gpu_lib.workspace_bytes("solve", gpu_lib.F32, 2497, 2497) > gpu_lib.NOALLOC_SCRATCH_BYTES
    _compare(gpu_lib, 2496, 2496, "f32", 5, "row")
    _compare(gpu_lib, 1000, 1500, "f32", 6, "row")


def test_noalloc_rejects_oversize(gpu_lib):
    # a float32 square just over the scratch
    d = 2600
    assert gpu_lib.workspace_bytes("solve", gpu_lib.F32, d, d) > gpu_lib.NOALLOC_SCRATCH_BYTES
    W = torch.zeros(d, d, device="cuda")
    LA = torch.eye(d, device="cuda")
    LB = torch.eye(d, device="cuda")
    V = torch.empty(d, d, dtype=torch.int32, device="cuda")
    with pytest.raises(gpu_lib.BakronError) as ei:
        gpu_lib.solve_noalloc(W, LA, LB, (0, 0, 1), None, V)
    assert ei.value.status == gpu_lib.EINVAL
