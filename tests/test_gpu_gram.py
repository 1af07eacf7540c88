"""GPU Kronecker-factor estimation (bakron_gram, bakron_sample_sqnorms)
against the oracle's weighted_gram / kfac_factors / shampoo_factors.

Tolerance, from the arithmetic: each entry is a sum over the N samples
accumulated in the dtype (one rounding per accumulation step, and one for
w_k x_kj when weights are given), so |G_gpu - G_ref| <= (N + 4) eps S with
S = (1/N) |X|^T |w| |X| (entrywise absolute values), plus eps |G| for the
final scaling and the damping. A dropped or repeated sample, a wrong weight
or a transposed index moves an entry by a whole term, far outside it at the
sizes used here."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import config3_samples

from parity_util import to_dev

pytestmark = pytest.mark.gpu

EPS = {np.float32: 2.0 ** -24, np.float64: 2.0 ** -53}


def _bound(X, w, Gref, dtype):
    Xa = np.abs(X.astype(np.float64))
    N = X.shape[0]
    S = (Xa.T @ (Xa * (np.abs(w)[:, None] if w is not None else 1.0))) / max(N, 1)
    eps = EPS[dtype]
    return (N + 4) * eps * S + 2 * eps * np.abs(Gref) + 1e-300


def _check(bk, X, w, damp, dtype):
    G = bk.gram(to_dev(X), None if w is None else to_dev(w), damp).cpu().numpy()
    assert np.array_equal(G, G.T), "not exactly symmetric"
    ref = O.damp(O.weighted_gram(X, w), damp)
    err = np.abs(G.astype(np.float64) - ref)
    tol = _bound(X, w, ref, dtype)
    assert np.all(err <= tol), (float(np.max(err / tol)), np.unravel_index(np.argmax(err / tol), err.shape))
    return G


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("N,d", [(1, 1), (37, 5), (100, 130), (513, 200), (16, 64), (3, 257),
                                 (1000, 1100)])
@pytest.mark.parametrize("weighted", [False, True])
def test_gram_matches_oracle(gpu_lib, dtype, N, d, weighted):
    rng = np.random.default_rng(N * 7 + d)
    X = (rng.standard_normal((N, d)) * rng.uniform(0.1, 3.0, d)).astype(dtype)
    w = rng.uniform(0.2, 5.0, N).astype(dtype) if weighted else None
    _check(gpu_lib, X, w, 0.01 if weighted else 0.0, dtype)


def test_gram_edge_cases(gpu_lib):
    bk = gpu_lib
    X = np.zeros((0, 9), np.float32)
    G = bk.gram(torch.zeros((0, 9), device="cuda"), None, 0.1).cpu().numpy()
    assert np.all(G == 0)
    # a leading dimension larger than d (a column slice of a wider buffer)
    base = np.random.default_rng(1).standard_normal((50, 80)).astype(np.float32)
    Xs = torch.from_numpy(base).cuda()[:, :70]
    G = bk.gram(Xs).cpu().numpy()
    ref = O.weighted_gram(base[:, :70])
    assert np.all(np.abs(G - ref) <= _bound(base[:, :70], None, ref, np.float32))


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_kfac_and_shampoo_factors(gpu_lib, dtype):
    bk = gpu_lib
    rng = np.random.default_rng(5)
    N, n, m = 300, 70, 50
    Xa = rng.standard_normal((N, n)).astype(dtype)
    Xb = (rng.standard_normal((N, m)) * (1 + np.abs(Xa[:, :1]))).astype(dtype)  # dependent sides
    sq = bk.sample_sqnorms(to_dev(Xb)).cpu().numpy()
    np.testing.assert_allclose(sq, O.sample_sqnorms(Xb), rtol=4 * EPS[dtype])
    A, B = bk.kfac_factors(to_dev(Xa), to_dev(Xb))
    Ar, Br = O.kfac_factors(Xa, Xb)
    for G, R, X in ((A, Ar, Xa), (B, Br, Xb)):
        assert np.all(np.abs(G.cpu().numpy() - R) <= _bound(X, None, R, dtype))
    A, B = bk.shampoo_factors(to_dev(Xa), to_dev(Xb))
    Ar, Br = O.shampoo_factors(Xa, Xb, iters=1)
    wa, wb = O.sample_sqnorms(Xb), O.sample_sqnorms(Xa)
    for G, R, X, w in ((A, Ar, Xa, wa), (B, Br, Xb, wb)):
        # the weights themselves carry one rounding to the dtype
        tol = _bound(X, w, R, dtype) + 2 * EPS[dtype] * np.abs(R)
        assert np.all(np.abs(G.cpu().numpy() - R) <= tol)


def test_gram_attn4096_activations(gpu_lib):
    """Config 3's input-side Gram at full size (8192 activations of 4096
    channels, 41 outlier channels x20, 1% mean-diagonal damping)."""
    bk = gpu_lib
    Xa, _ = config3_samples()
    G = _check(bk, Xa, None, 1e-2, np.float32)
    assert G.shape == (4096, 4096)
