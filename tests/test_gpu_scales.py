"""GPU per-row scale search (bakron_row_scales_mse) against the oracle's
row_scales_mse: the same candidate chosen on every row, except where two
candidates' errors are equal to float64 summation-order precision (then the
GPU's choice must attain the oracle's minimum error)."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import config3

from parity_util import to_dev

pytestmark = pytest.mark.gpu


def _check(bk, W, alphabet, grid, shrink, rows=None):
    lo, hi = alphabet
    s_gpu = bk.row_scales_mse(to_dev(W), (lo, hi, 0), grid, shrink).cpu().numpy()
    idx = np.arange(W.shape[0]) if rows is None else rows
    Ws = W[idx]
    s_ref = O.row_scales_mse(Ws, lo, hi, grid, shrink, W.dtype)
    s_gpu = s_gpu[idx]
    diff = np.nonzero(s_gpu != s_ref)[0]
    if len(diff):
        e_gpu = O.row_rtn_error(Ws[diff], s_gpu[diff], lo, hi)
        e_ref = O.row_rtn_error(Ws[diff], s_ref[diff], lo, hi)
        np.testing.assert_allclose(e_gpu, e_ref, rtol=1e-12)
    assert len(diff) <= max(1, len(idx) // 1000), (len(diff), len(idx))
    # the chosen scale is one of the candidates of its row
    smax = O.row_scales(Ws, hi, W.dtype)
    for i in range(min(len(idx), 20)):
        if smax[i] == 1 and not np.any(Ws[i]):
            assert s_gpu[i] == 1
            continue
        cands = {W.dtype.type(np.float64(smax[i]) * O.shrink_factor(k, grid, shrink))
                 for k in range(grid + 1)}
        assert s_gpu[i] in cands
    return s_gpu


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("m,n", [(1, 1), (7, 300), (33, 1000), (64, 4099)])
@pytest.mark.parametrize("alphabet", [(-8, 7), (-4, 3), (-3, 3)])
def test_scale_search_matches_oracle(gpu_lib, dtype, m, n, alphabet):
    rng = np.random.default_rng(m * 1000 + n + alphabet[1])
    W = (rng.standard_t(4, (m, n)) * 0.02).astype(dtype)
    if m > 3:
        W[2] = 0.0  # all-zero row: scale 1
    _check(gpu_lib, W, alphabet, 100, 0.5)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_scale_search_without_search_is_absmax(gpu_lib, dtype):
    bk = gpu_lib
    W = (np.random.default_rng(5).standard_normal((50, 333)) * 0.02).astype(dtype)
    W[7] = 0.0
    plain = bk.row_scales(to_dev(W), 7)
    for grid, shrink in ((0, 0.5), (40, 0.0)):
        s = bk.row_scales_mse(to_dev(W), (-8, 7, 0), grid, shrink)
        assert torch.equal(s, plain)


def test_scale_search_grids(gpu_lib):
    """Grid sizes below, at and above one candidate chunk, up to the maximum."""
    W = (np.random.default_rng(6).standard_t(3, (9, 517)) * 0.02).astype(np.float32)
    for grid in (1, 15, 16, 17, 1024):
        _check(gpu_lib, W, (-8, 7), grid, 0.5)
    _check(gpu_lib, W, (-8, 7), 64, 0.75)


def test_scale_search_attn4096(gpu_lib):
    """The 4096 x 4096 weight at full size; 512 sampled rows against the oracle."""
    W = config3().W
    rows = np.random.default_rng(7).choice(W.shape[0], 512, replace=False)
    s = _check(gpu_lib, W, (-8, 7), 100, 0.5, rows=np.sort(rows))
    assert np.all(s > 0)
