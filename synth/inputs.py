"""Seeded synthetic inputs for the BaKron solver.

This module only draws random numbers and assembles the Gram matrices that
stand in for Hessian factors; it holds none of the solver's arithmetic
(no factorisation, no rounding, no scale rule). Both the CPU oracle and the
GPU path consume what it returns, so it is the one module they share.

Source of the workload shapes: "BaKron: Efficient Quantization with
Kronecker-Factored Hessians" (arXiv 2608.06291), §6 Table 3 (the benchmark
shapes, square up to 8192 and the Llama-3-8B MLP shapes 14336x4096 /
4096x14336) and §4 / Appendix D (A is an input-side Gram, B an output-side
Gram, each regularised by adding a multiple of the identity). The pages give
no Hessians for the timing table, so the distributions below are our own
stand-ins; every recipe is spelled out in the function that builds it.

Seeds: ``numpy.random.default_rng([config_id, matrix_idx, role])`` with roles
W=0, input-side samples=1, output-side samples=2, outlier pick=3.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

ROLE_W, ROLE_A, ROLE_B, ROLE_OUTLIER = 0, 1, 2, 3


def rng(config_id: int, matrix_idx: int, role: int) -> np.random.Generator:
    return np.random.default_rng([int(config_id), int(matrix_idx), int(role)])


@dataclass
class Problem:
    """One quantisation problem: W (m x n), A (n x n), B (m x m).

    ``alphabet`` is (lo, hi, unbounded). ``scale_hi`` is the divisor of the
    per-row absmax scale rule (7 for {-8..7}, 3 for {-4..3}); None means no
    scales (plain rounding to the integers).
    """
    name: str
    W: np.ndarray
    A: np.ndarray
    B: np.ndarray
    dtype: str                      # "f32" or "f64": the solver's mode
    alphabet: tuple = (0, 0, 1)     # (lo, hi, unbounded)
    scale_hi: Optional[int] = None  # per-row absmax / scale_hi, or None
    meta: dict = field(default_factory=dict)

    @property
    def m(self) -> int:
        return self.W.shape[0]

    @property
    def n(self) -> int:
        return self.W.shape[1]

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.float64


def gram(X: np.ndarray, damp_rel: float = 0.0, damp_abs: float = 0.0) -> np.ndarray:
    """G = X X^T / N (N = number of columns), then + (damp_rel*mean(diag G) + damp_abs) I."""
    N = X.shape[1]
    G = (X @ X.T) / float(N)
    G = 0.5 * (G + G.T)
    d = damp_rel * float(np.mean(np.diag(G))) + damp_abs
    if d:
        G[np.diag_indices_from(G)] += d
    return G


def _gaussian(g: np.random.Generator, shape, dtype=np.float64) -> np.ndarray:
    return g.standard_normal(shape, dtype=dtype)


def wishart_gram(g: np.random.Generator, dim: int, samples: int, damp_rel: float = 1e-2,
                 sample_dtype=np.float64) -> np.ndarray:
    X = _gaussian(g, (dim, samples), sample_dtype)
    return gram(X, damp_rel=damp_rel).astype(np.float64)


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------

def config1(matrix_idx: int = 0) -> Problem:
    """64x64, fp64. W = 2*N(0,1). A = X X^T/256 + 1e-2 I with X ~ N(0,1) 64x256;
    B built the same way from an independent seed. Alphabet: all integers."""
    cid = 1
    W = 2.0 * _gaussian(rng(cid, matrix_idx, ROLE_W), (64, 64))
    A = gram(_gaussian(rng(cid, matrix_idx, ROLE_A), (64, 256)), damp_abs=1e-2)
    B = gram(_gaussian(rng(cid, matrix_idx, ROLE_B), (64, 256)), damp_abs=1e-2)
    return Problem("cfg1_64x64_f64", W, A, B, "f64", (0, 0, 1), None)


def config2(matrix_idx: int = 0) -> Problem:
    """512x512, fp32. W ~ N(0, 0.02^2). A = Gram/2048 of 2048 activations whose
    channel c has scale sigma_c = |t_4| (Student-t, 4 dof) times N(0,1) noise;
    B = Gram/2048 of 2048 N(0,I) output-gradient vectors. Both damped by
    1e-2*mean(diag). 4-bit alphabet {-8..7} with per-row absmax/7 scales."""
    cid, m, n, N = 2, 512, 512, 2048
    W = 0.02 * _gaussian(rng(cid, matrix_idx, ROLE_W), (m, n))
    ga = rng(cid, matrix_idx, ROLE_A)
    sigma = np.abs(ga.standard_t(4, size=n))
    XA = sigma[:, None] * _gaussian(ga, (n, N))
    A = gram(XA, damp_rel=1e-2)
    B = gram(_gaussian(rng(cid, matrix_idx, ROLE_B), (m, N)), damp_rel=1e-2)
    return Problem("cfg2_512x512_f32", W.astype(np.float32), A.astype(np.float32),
                   B.astype(np.float32), "f32", (-8, 7, 0), 7)


def config3_samples(matrix_idx: int = 0):
    """The samples behind config 3's Grams, one sample per ROW (N x dim,
    float32): the 8192 activations (with the 41 outlier channels x20) and the
    8192 gradient vectors, drawn exactly as config3 draws them."""
    cid, m, n, N = 3, 4096, 4096, 8192
    XA = _gaussian(rng(cid, matrix_idx, ROLE_A), (n, N), np.float32)
    n_out = int(round(0.01 * n))
    out = rng(cid, matrix_idx, ROLE_OUTLIER).choice(n, size=n_out, replace=False)
    XA[out, :] *= 20.0
    XB = _gaussian(rng(cid, matrix_idx, ROLE_B), (m, N), np.float32)
    return np.ascontiguousarray(XA.T), np.ascontiguousarray(XB.T)


def config3(matrix_idx: int = 0) -> Problem:
    """4096x4096 fp32 (Llama-3-8B attention projection shape). W ~ N(0,0.02^2).
    A = Gram/8192 of 8192 N(0,I) activations in which round(1% of n) = 41
    channels (seeded pick) are multiplied by 20; B = Gram/8192 of 8192 N(0,I)
    gradient vectors. Both damped by 1% of the mean diagonal. 4-bit per-row
    absmax/7 scales."""
    cid, m, n, N = 3, 4096, 4096, 8192
    W = 0.02 * _gaussian(rng(cid, matrix_idx, ROLE_W), (m, n), np.float32)
    XA = _gaussian(rng(cid, matrix_idx, ROLE_A), (n, N), np.float32)
    n_out = int(round(0.01 * n))
    out = rng(cid, matrix_idx, ROLE_OUTLIER).choice(n, size=n_out, replace=False)
    XA[out, :] *= 20.0
    A = gram(XA.astype(np.float64), damp_rel=1e-2)
    del XA
    XB = _gaussian(rng(cid, matrix_idx, ROLE_B), (m, N), np.float32).astype(np.float64)
    B = gram(XB, damp_rel=1e-2)
    del XB
    return Problem("cfg3_4096x4096_f32", W.astype(np.float32), A.astype(np.float32),
                   B.astype(np.float32), "f32", (-8, 7, 0), 7,
                   meta={"outlier_channels": np.sort(out)})


def config4(which: str = "gate_up", matrix_idx: int = 0) -> Problem:
    """Llama-3-8B MLP shapes, fp32: gate/up m=14336,n=4096 or down m=4096,n=14336.
    W ~ N(0,0.02^2); A (n x n) and B (m x m) are Grams/16384 of 16384 N(0,I)
    samples, damped by 1% of the mean diagonal; 3-bit alphabet {-4..3} with
    per-row absmax/3 scales. The samples are drawn in fp32 and the Gram is
    accumulated in fp32 (sgemm) to keep generation to seconds; the result is
    an SPD matrix either way and both sides receive the same one."""
    cid = 4
    if which == "gate_up":
        m, n, sub = 14336, 4096, 0
    elif which == "down":
        m, n, sub = 4096, 14336, 1
    else:
        raise ValueError(which)
    N = 16384
    mi = 2 * matrix_idx + sub
    W = 0.02 * _gaussian(rng(cid, mi, ROLE_W), (m, n), np.float32)
    XA = _gaussian(rng(cid, mi, ROLE_A), (n, N), np.float32)
    A = gram(XA, damp_rel=1e-2)
    del XA
    XB = _gaussian(rng(cid, mi, ROLE_B), (m, N), np.float32)
    B = gram(XB, damp_rel=1e-2)
    del XB
    return Problem(f"cfg4_{which}_{m}x{n}_f32", W.astype(np.float32), A.astype(np.float32),
                   B.astype(np.float32), "f32", (-4, 3, 0), 3)


def config5(matrix_idx: int, b_identity: bool = False) -> Problem:
    """One of 28 small-model k/v projections, m=1024, n=2048, fp32.
    A, B = Wishart(4096 dof)/4096 + 1% mean-diag damping (B = I when
    ``b_identity``, the one-sided GPTQ case). 4-bit per-row absmax/7 scales."""
    cid, m, n, N = 5, 1024, 2048, 4096
    W = 0.02 * _gaussian(rng(cid, matrix_idx, ROLE_W), (m, n))
    A = wishart_gram(rng(cid, matrix_idx, ROLE_A), n, N)
    if b_identity:
        B = np.eye(m)
    else:
        B = wishart_gram(rng(cid, matrix_idx, ROLE_B), m, N)
    name = f"cfg5_{matrix_idx}_{m}x{n}_f32" + ("_BI" if b_identity else "")
    return Problem(name, W.astype(np.float32), A.astype(np.float32), B.astype(np.float32),
                   "f32", (-8, 7, 0), 7)


def head_grams(config_id: int, heads: int, b: int, samples: int, damp_rel: float = 1e-2,
               dtype=np.float64) -> np.ndarray:
    """Per-head output-side Grams, (heads, b, b): head h is the Gram/N of
    ``samples`` N(0, I) vectors of dimension b (seed [config_id, h, ROLE_B]),
    damped by ``damp_rel`` of its mean diagonal. Stand-ins for the per-head
    attention-local output factors the pages assemble block-diagonally."""
    out = np.empty((heads, b, b), dtype=np.float64)
    for h in range(heads):
        out[h] = gram(_gaussian(rng(config_id, h, ROLE_B), (b, samples)), damp_rel=damp_rel)
    return out.astype(dtype)


def block_diag(blocks: np.ndarray) -> np.ndarray:
    """The (h b) x (h b) matrix with the given (h, b, b) blocks on its diagonal."""
    h, b, _ = blocks.shape
    M = np.zeros((h * b, h * b), dtype=blocks.dtype)
    for i in range(h):
        M[i * b:(i + 1) * b, i * b:(i + 1) * b] = blocks[i]
    return M


def config3_heads(heads: int = 32, base: Optional[Problem] = None) -> tuple:
    """The 4096 x 4096 attention workload with a block-diagonal output side:
    W and A of ``config3`` (or of ``base``), and B = blockdiag of ``heads``
    per-head Grams (b = 4096 / heads = 128 for 32 heads) of 8192 Gaussian
    output vectors each, 1% damping. Returns (problem with the assembled
    dense B, the (heads, b, b) blocks)."""
    p = base if base is not None else config3()
    m = p.W.shape[0]
    b = m // heads
    blocks = head_grams(6, heads, b, 8192).astype(np.float32)
    q = Problem(f"cfg3_heads{heads}_{m}x{p.W.shape[1]}_f32", p.W, p.A, block_diag(blocks), p.dtype,
                p.alphabet, p.scale_hi, meta={"heads": heads})
    return q, blocks


# ---------------------------------------------------------------------------
# Generic small problems for tests (any shape / dtype / alphabet).
# ---------------------------------------------------------------------------

def random_problem(m: int, n: int, dtype: str = "f64", seed: int = 0, samples_factor: int = 4,
                   damp_rel: float = 1e-2, alphabet=(0, 0, 1), scale_hi=None,
                   w_std: float = 2.0, heavy_tail: bool = False) -> Problem:
    """Wishart-style A (n x n) and B (m x m) from seed ``seed`` with
    ``samples_factor * dim`` samples, 1% mean-diag damping by default.
    ``heavy_tail`` gives input channels Student-t(4) scales as in the
    512x512 workload."""
    g = np.random.default_rng([100, int(seed), int(m), int(n)])
    W = w_std * g.standard_normal((m, n))
    NA = max(1, samples_factor * n)
    XA = g.standard_normal((n, NA))
    if heavy_tail:
        XA *= np.abs(g.standard_t(4, size=n))[:, None]
    A = gram(XA, damp_rel=damp_rel)
    NB = max(1, samples_factor * m)
    B = gram(g.standard_normal((m, NB)), damp_rel=damp_rel)
    npdt = np.float32 if dtype == "f32" else np.float64
    return Problem(f"rand_{m}x{n}_{dtype}_s{seed}", W.astype(npdt), A.astype(npdt), B.astype(npdt),
                   dtype, tuple(alphabet), scale_hi)


CONFIGS = {
    1: config1,
    2: config2,
    3: config3,
}
