"""CPU oracle for the BaKron solver (float64).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run anything under ``oracle/``.
The GPU library never links, imports or calls it, and it imports nothing from
the GPU package; the two share no code.

Everything here follows "BaKron: Efficient Quantization with
Kronecker-Factored Hessians" (arXiv 2608.06291). Section references below are
to that page. All arithmetic is float64; float32 inputs are upcast exactly.

What is computed (the plain definition, Appendix B, recurrence (2)):
with normalised unit-lower factors L^A = Cholesky(A^-1), L^B = Cholesky(B^-1)
(columns divided by their diagonals), the value at which entry (p,q) is
rounded is W0[p,q] plus the errors of all entries (i,j) != (p,q) with i<=p
and j<=q, each weighted by L^B[p,i] L^A[q,j]. ``solve_naive`` evaluates this
entry by entry (Algorithm 2); ``solve_antidiag`` (Algorithm 3),
``solve_recursive`` (Algorithm 5) and ``solve_bakron`` (Algorithm 6) are the
reorderings that Theorem 3.2 proves equal. ``solve_recursive`` with a plain-C
naive leaf is the fast oracle used at large sizes.

Readings of points the pages leave open:
* ties in rounding go to even (``rint``); Appendix B only says a rule is fixed;
* quantize(x) = clamp(rint(x / s), lo, hi) with a true division by the
  entry's row (or column) scale; unbounded alphabets use rint(x / s);
* the factor is taken literally: inverse, then Cholesky (§3.2, Algorithm 2);
* only the lower triangles of A and B are read (they are symmetric);
* recursive calls work in place on one workspace and the factorisation is
  done once at the top (Appendix B, conventions for the recursive
  algorithms); midpoints are floor((k+l)/2).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

from . import build as _build

SCALE_NONE, SCALE_ROW, SCALE_COL = 0, 1, 2


# ---------------------------------------------------------------------------
# Small helpers
# ---------------------------------------------------------------------------

def sym_from_lower(A: np.ndarray) -> np.ndarray:
    """The symmetric matrix whose lower triangle is that of A."""
    A = np.asarray(A, dtype=np.float64)
    return np.tril(A) + np.tril(A, -1).T


def vec(W: np.ndarray) -> np.ndarray:
    """Column-major flattening (§3.1): vec(W)[j*m + i] = W[i, j]."""
    return np.asarray(W).reshape(-1, order="F")


def unvec(v: np.ndarray, m: int, n: int) -> np.ndarray:
    return np.asarray(v).reshape((m, n), order="F")


@dataclass
class Alphabet:
    """{lo, ..., hi} or all integers (unbounded). §3.1: alphabet {-2^b..2^b-1}."""
    lo: int = 0
    hi: int = 0
    unbounded: bool = True

    @staticmethod
    def of(t) -> "Alphabet":
        if isinstance(t, Alphabet):
            return t
        lo, hi, unb = t
        return Alphabet(int(lo), int(hi), bool(unb))


def quantize(x, s, alphabet) -> np.ndarray:
    """§3.1: replace round by a quantizer mapping x to the closest alphabet
    element after scaling by s. Codes are returned as float64 integers."""
    al = Alphabet.of(alphabet)
    c = np.rint(np.asarray(x, dtype=np.float64) / np.asarray(s, dtype=np.float64))
    if not al.unbounded:
        c = np.clip(c, al.lo, al.hi)
    return c


def scale_grid(m: int, n: int, scale_mode: int, scales) -> np.ndarray:
    """Per-entry scale s[i,j] from per-row / per-column scales (§3.1)."""
    if scale_mode == SCALE_NONE:
        return np.ones((m, n))
    s = np.asarray(scales, dtype=np.float64)
    if scale_mode == SCALE_ROW:
        assert s.shape == (m,)
        return np.broadcast_to(s[:, None], (m, n)).copy()
    if scale_mode == SCALE_COL:
        assert s.shape == (n,)
        return np.broadcast_to(s[None, :], (m, n)).copy()
    raise ValueError(scale_mode)


def row_scales(W: np.ndarray, hi: int, dtype=None) -> np.ndarray:
    """Per-row absmax scale: s_i = max_j |W_ij| / hi, and 1 where the row is 0.
    Appendix D chooses per-row scales as absmax divided by the largest code.
    Computed in ``dtype`` (default: W's dtype) so both sides of a parity test
    receive the same float."""
    W = np.asarray(W)
    dt = np.dtype(dtype) if dtype is not None else W.dtype
    amax = np.max(np.abs(W), axis=1).astype(dt)
    s = amax / dt.type(hi)
    s[amax == 0] = dt.type(1)
    return s.astype(dt)


def shrink_factor(k: int, grid: int, max_shrink: float) -> float:
    """Candidate k of the scale search: 1 - max_shrink * k / grid, evaluated
    in float64 in exactly this order (max_shrink * k, then / grid, then
    1 - that), so that every implementation forms the same candidates."""
    if grid == 0:
        return 1.0
    return 1.0 - (float(max_shrink) * float(k)) / float(grid)


def row_scales_mse(W: np.ndarray, lo: int, hi: int, grid: int, max_shrink: float,
                   dtype=None) -> np.ndarray:
    """Per-row scale search of Appendix D (experimental setup): start from the
    row's absmax divided by the largest code, then shrink it by up to a
    factor 1 / (1 - max_shrink) (the pages: up to 2, max_shrink = 1/2)
    choosing the candidate with the smallest round-to-nearest squared error
    of the row. Reading of the unspecified search: grid + 1 candidates
    s_k = s_max * (1 - max_shrink * k / grid), k = 0..grid (product in
    float64, rounded once to ``dtype``); the row's error for s_k is
    sum_j (W_ij - s_k c_j)^2 with c_j = clamp(rint(W_ij / s_k), lo, hi) (the
    quantizer of §3.1, division in ``dtype``), summed in float64; the
    smallest error wins and ties go to the smaller k (the larger scale). An
    all-zero row keeps the scale 1 of the plain rule."""
    W = np.asarray(W)
    dt = np.dtype(dtype) if dtype is not None else W.dtype
    Wd = W.astype(dt)
    base = row_scales(Wd, hi, dt)
    out = base.copy()
    for i in range(Wd.shape[0]):
        row = Wd[i]
        if not np.any(row != 0):
            continue
        best, best_s = None, base[i]
        for k in range(grid + 1):
            sk = dt.type(np.float64(base[i]) * shrink_factor(k, grid, max_shrink))
            c = np.clip(np.rint(row / sk), lo, hi)
            e = row.astype(np.float64) - np.float64(sk) * c.astype(np.float64)
            err = float(np.sum(e * e))
            if best is None or err < best:
                best, best_s = err, sk
        out[i] = best_s
    return out.astype(dt)


def row_rtn_error(W: np.ndarray, s: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Per-row squared round-to-nearest error sum_j (W_ij - s_i c_ij)^2,
    c = clamp(rint(W / s), lo, hi), in float64 (division in W's dtype)."""
    W = np.asarray(W)
    c = np.clip(np.rint(W / s[:, None].astype(W.dtype)), lo, hi)
    e = W.astype(np.float64) - s[:, None].astype(np.float64) * c
    return np.sum(e * e, axis=1)


# ---------------------------------------------------------------------------
# Kronecker factors from samples (§4.2, Appendix A.2)
# ---------------------------------------------------------------------------

def weighted_gram(X: np.ndarray, w: Optional[np.ndarray] = None) -> np.ndarray:
    """(1/N) sum_k w_k x_k x_k^T over the N rows x_k of X (w = 1 when None),
    in float64: the sample expectation E[w x x^T]."""
    X = np.asarray(X, dtype=np.float64)
    N = X.shape[0]
    if N == 0:
        return np.zeros((X.shape[1], X.shape[1]))
    Xw = X if w is None else X * np.asarray(w, dtype=np.float64)[:, None]
    return (X.T @ Xw) / N


def damp(G: np.ndarray, rel: float) -> np.ndarray:
    """G + rel * mean(diag(G)) * I: the Gram regularisation of the
    experiments (Appendix D adds a multiple of the mean diagonal)."""
    G = np.array(G, dtype=np.float64)
    if G.shape[0]:
        G[np.diag_indices_from(G)] += rel * float(np.mean(np.diag(G)))
    return G


def kfac_factors(Xa: np.ndarray, Xb: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """K-FAC-style factors (§4.2: independence pulls the expectation apart):
    H = E[a a^T (x) b b^T] ~ E[a a^T] (x) E[b b^T]; sample k is row k of Xa
    (input side, n) and of Xb (output side, m)."""
    return weighted_gram(Xa), weighted_gram(Xb)


def shampoo_factors(Xa: np.ndarray, Xb: np.ndarray, iters: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Shampoo-style factors (§4.2, Appendix A.2): the power iteration for the
    top singular vectors of the rearranged Hessian, written on the factors,
    from A = I, B = I: both new factors from the previous pair,
        A' = E[(b^T B b) a a^T],   B' = E[(a^T A a) b b^T],
    without normalisation (the solver is invariant to scaling either factor).
    One iteration gives E[|b|^2 a a^T] and E[|a|^2 b b^T]."""
    Xa = np.asarray(Xa, dtype=np.float64)
    Xb = np.asarray(Xb, dtype=np.float64)
    A = np.eye(Xa.shape[1])
    B = np.eye(Xb.shape[1])
    for it in range(iters):
        if it > 0:  # keep many iterations finite; the scale is irrelevant
            A, B = A / np.linalg.norm(A), B / np.linalg.norm(B)
        wa = np.einsum("ki,ij,kj->k", Xb, B, Xb)  # b_k^T B b_k
        wb = np.einsum("ki,ij,kj->k", Xa, A, Xa)  # a_k^T A a_k
        A, B = weighted_gram(Xa, wa), weighted_gram(Xb, wb)
    return A, B


def sample_sqnorms(X: np.ndarray) -> np.ndarray:
    """|x_k|^2 of every row, in float64 (the one-step Shampoo weights)."""
    X = np.asarray(X, dtype=np.float64)
    return np.sum(X * X, axis=1)


# ---------------------------------------------------------------------------
# Factor (first two steps of Algorithms 1-3, 5, 6)
# ---------------------------------------------------------------------------

def factor(A: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """L = Cholesky(A^-1) (§3.1: lower triangular, L L^T = A^-1, positive
    diagonal), then each column divided by its diagonal entry (§3.2,
    Algorithm 1 and 2). Returns (Lhat, d) with d = diag(L).

    Raises numpy.linalg.LinAlgError when A is not (numerically) positive
    definite."""
    A = sym_from_lower(A)
    if not np.all(np.isfinite(A)):
        raise np.linalg.LinAlgError("non-finite entries")
    Ainv = np.linalg.inv(A)
    L = np.linalg.cholesky(Ainv)
    d = np.diag(L).copy()
    Lhat = L / d[None, :]
    return Lhat, d


def rev_cholesky(A: np.ndarray) -> np.ndarray:
    """RevCholesky (§3.1): the lower triangular R with R^T R = A and positive
    diagonal, computed through the reversal permutation J: Cholesky(J A J) =
    J R^T J. Used only to check the error bound of Corollary 3.4."""
    A = sym_from_lower(A)
    C = np.linalg.cholesky(A[::-1, ::-1])
    return C.T[::-1, ::-1].copy()


# ---------------------------------------------------------------------------
# Algorithm 1 on a single vector with an explicit Hessian
# ---------------------------------------------------------------------------

def gptq_vector(w: np.ndarray, H: np.ndarray, s, alphabet) -> Tuple[np.ndarray, np.ndarray]:
    """§3.2, Algorithm 1 (GPTQ on one neuron) with a general Hessian H and
    per-coordinate scales s. Returns (codes, values at rounding time)."""
    w = np.array(w, dtype=np.float64)
    L, _ = factor(H)
    n = w.shape[0]
    s = np.broadcast_to(np.asarray(s, dtype=np.float64), (n,))
    codes = np.zeros(n)
    wt = np.zeros(n)
    for i in range(n):
        wt[i] = w[i]
        c = quantize(w[i], s[i], alphabet)
        codes[i] = c
        delta = s[i] * c - w[i]
        w = w + delta * L[:, i]
    return codes, wt


# ---------------------------------------------------------------------------
# Algorithm 2 (BaKron-naive): plain C loop, and a pure-Python twin for tiny cases
# ---------------------------------------------------------------------------

_lib = None


def _clib():
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.bk_oracle_naive.argtypes = [i64, i64, d, i64, d, i64, d, i64, d, d,
                                        ctypes.c_double, ctypes.c_double, ctypes.c_int,
                                        d, i64, d, i64, d, i64, d, i64, ctypes.c_int]
        lib.bk_oracle_naive.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.strides[-1] == 8
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _naive_block(W, LA, LB, srow, scol, al: Alphabet, forced, C, Wt, E, order=0):
    """Run the C naive loop on views (all float64, last stride 8)."""
    m, n = W.shape
    if m == 0 or n == 0:
        return
    lib = _clib()
    rc = lib.bk_oracle_naive(
        m, n, _ptr(W), W.strides[0] // 8, _ptr(LA), LA.strides[0] // 8, _ptr(LB), LB.strides[0] // 8,
        _ptr(srow), _ptr(scol), float(al.lo), float(al.hi), int(al.unbounded),
        _ptr(forced), (forced.strides[0] // 8) if forced is not None else 0,
        _ptr(C), C.strides[0] // 8, _ptr(Wt), Wt.strides[0] // 8, _ptr(E), E.strides[0] // 8, int(order))
    if rc != 0:
        raise RuntimeError("bk_oracle_naive failed")


@dataclass
class Result:
    V: np.ndarray        # codes (float64 integers)
    Wt: np.ndarray       # value of each entry when it was rounded
    E: np.ndarray        # error s*V - Wt

    def codes_int(self) -> np.ndarray:
        return self.V.astype(np.int64)


def _prep(W, LA, LB, scale_mode, scales):
    W = np.array(W, dtype=np.float64, order="C")
    LA = np.ascontiguousarray(LA, dtype=np.float64)
    LB = np.ascontiguousarray(LB, dtype=np.float64)
    m, n = W.shape
    assert LA.shape == (n, n) and LB.shape == (m, m)
    srow = scol = None
    if scale_mode == SCALE_ROW:
        srow = np.ascontiguousarray(scales, dtype=np.float64)
        assert srow.shape == (m,)
    elif scale_mode == SCALE_COL:
        scol = np.ascontiguousarray(scales, dtype=np.float64)
        assert scol.shape == (n,)
    return W, LA, LB, srow, scol


def solve_naive(W, LA, LB, alphabet, scale_mode=SCALE_NONE, scales=None, order: str = "col",
                forced=None) -> Result:
    """§3.2 Algorithm 2 in float64 (plain C loop). ``order`` "col" is the
    column-major vec order, "row" the row-major order the listing prints."""
    W, LA, LB, srow, scol = _prep(W, LA, LB, scale_mode, scales)
    m, n = W.shape
    C = np.zeros((m, n)); Wt = np.zeros((m, n)); E = np.zeros((m, n))
    f = None if forced is None else np.ascontiguousarray(forced, dtype=np.float64)
    _naive_block(W, LA, LB, srow, scol, Alphabet.of(alphabet), f, C, Wt, E,
                 order=0 if order == "col" else 1)
    return Result(C, Wt, E)


def solve_naive_py(W, LA, LB, alphabet, scale_mode=SCALE_NONE, scales=None, order="col") -> Result:
    """Pure-Python twin of ``solve_naive`` for tiny inputs: Algorithm 2 with
    the whole-matrix rank-1 update W <- W + L^B_i * delta * (L^A_j)^T."""
    W = np.array(W, dtype=np.float64)
    LA = np.asarray(LA, dtype=np.float64)
    LB = np.asarray(LB, dtype=np.float64)
    m, n = W.shape
    S = scale_grid(m, n, scale_mode, scales)
    C = np.zeros((m, n)); Wt = np.zeros((m, n)); E = np.zeros((m, n))
    idx = [(i, j) for j in range(n) for i in range(m)] if order == "col" else \
          [(i, j) for i in range(m) for j in range(n)]
    for (i, j) in idx:
        x = W[i, j]
        c = quantize(x, S[i, j], alphabet)
        delta = S[i, j] * c - x
        C[i, j], Wt[i, j], E[i, j] = c, x, delta
        W = W + np.outer(LB[:, i], LA[:, j]) * delta
    return Result(C, Wt, E)


# ---------------------------------------------------------------------------
# Algorithm 3 (BaKron-antidiagonal)
# ---------------------------------------------------------------------------

def antidiag_mask(m: int, n: int, k0: int, k1: Optional[int] = None) -> np.ndarray:
    """Boolean mask of anti-diagonals k0 <= i+j < k1 (0-based: i+j runs from 0
    to m+n-2; the pages count from 2 with 1-based indices, §3.1)."""
    if k1 is None:
        k1 = k0 + 1
    ii, jj = np.indices((m, n))
    s = ii + jj
    return (s >= k0) & (s < k1)


def solve_antidiag(W, LA, LB, alphabet, scale_mode=SCALE_NONE, scales=None) -> Result:
    """§3.3 Algorithm 3: for each anti-diagonal, round all of its entries at
    once, then W <- W + L^B Delta (L^A)^T with Delta the errors on it."""
    W = np.array(W, dtype=np.float64)
    LA = np.asarray(LA, dtype=np.float64)
    LB = np.asarray(LB, dtype=np.float64)
    m, n = W.shape
    S = scale_grid(m, n, scale_mode, scales)
    C = np.zeros((m, n)); Wt = np.zeros((m, n)); E = np.zeros((m, n))
    for k in range(m + n - 1):
        mk = antidiag_mask(m, n, k)
        D = np.where(mk, W, 0.0)
        c = quantize(D, S, alphabet)
        delta = np.where(mk, S * c - D, 0.0)
        C[mk], Wt[mk], E[mk] = c[mk], D[mk], delta[mk]
        W = W + LB @ delta @ LA.T
    return Result(C, Wt, E)


# ---------------------------------------------------------------------------
# Algorithm 6 (BaKron): recursion over ranges of anti-diagonals, numpy
# ---------------------------------------------------------------------------

def solve_bakron(W, LA, LB, alphabet, scale_mode=SCALE_NONE, scales=None) -> Result:
    """§3.5 Algorithm 6 at entry granularity: process anti-diagonals [k, mid)
    recursively, add antidiag_{mid:l}(L^B (V - antidiag_{k:mid}(W)) (L^A)^T)
    to the workspace, then process [mid, l). The workspace keeps each
    entry's pre-rounding value (Appendix B conventions), so V - W on the
    processed band is the error matrix E. Dense products; for small inputs."""
    W = np.array(W, dtype=np.float64)
    LA = np.asarray(LA, dtype=np.float64)
    LB = np.asarray(LB, dtype=np.float64)
    m, n = W.shape
    S = scale_grid(m, n, scale_mode, scales)
    C = np.zeros((m, n)); Wt = np.zeros((m, n)); E = np.zeros((m, n))

    def rec(k: int, l: int):
        if l == k + 1:
            mk = antidiag_mask(m, n, k)
            c = quantize(W[mk], S[mk], alphabet)
            C[mk] = c
            Wt[mk] = W[mk]
            E[mk] = S[mk] * c - W[mk]
            return
        mid = (k + l) // 2
        rec(k, mid)
        Eband = np.where(antidiag_mask(m, n, k, mid), E, 0.0)
        U = LB @ Eband @ LA.T
        tgt = antidiag_mask(m, n, mid, l)
        W[tgt] += U[tgt]
        rec(mid, l)

    if m and n:
        rec(0, m + n - 1)
    return Result(C, Wt, E)


# ---------------------------------------------------------------------------
# Algorithm 5 (BaKron-recursive): the fast oracle
# ---------------------------------------------------------------------------

def solve_recursive(W, LA, LB, alphabet, scale_mode=SCALE_NONE, scales=None, leaf: int = 32,
                    forced=None) -> Result:
    """§3.4 Algorithm 5 in float64: split the longer side in half, solve the
    first half, add L^B (V - W)_{first half} (L^A)^T restricted to the second
    half, solve the second half. Factors are sliced from the top-level ones
    (Appendix B conventions). Blocks with both sides <= ``leaf`` run the
    plain-C Algorithm 2 loop on their own sub-factors; splitting stops there
    but the computation is the same recursion (a block solved by Algorithm 2
    equals the block solved by further splitting, Theorem 3.2).

    ``forced`` imposes codes instead of rounding (used to re-run recurrence
    (2) of Appendix B with given codes)."""
    W, LA, LB, srow, scol = _prep(W, LA, LB, scale_mode, scales)
    m, n = W.shape
    al = Alphabet.of(alphabet)
    C = np.zeros((m, n)); Wt = np.zeros((m, n)); E = np.zeros((m, n))
    F = None if forced is None else np.ascontiguousarray(forced, dtype=np.float64)

    def rec(i0, i1, j0, j1):
        mb, nb = i1 - i0, j1 - j0
        if mb <= 0 or nb <= 0:
            return
        if mb <= leaf and nb <= leaf:
            _naive_block(W[i0:i1, j0:j1], LA[j0:j1, j0:j1], LB[i0:i1, i0:i1],
                         None if srow is None else srow[i0:i1],
                         None if scol is None else scol[j0:j1], al,
                         None if F is None else F[i0:i1, j0:j1],
                         C[i0:i1, j0:j1], Wt[i0:i1, j0:j1], E[i0:i1, j0:j1], order=0)
            return
        if mb < nb:
            jm = j0 + nb // 2
            rec(i0, i1, j0, jm)
            W[i0:i1, jm:j1] += (LB[i0:i1, i0:i1] @ E[i0:i1, j0:jm]) @ LA[jm:j1, j0:jm].T
            rec(i0, i1, jm, j1)
        else:
            im = i0 + mb // 2
            rec(i0, im, j0, j1)
            W[im:i1, j0:j1] += (LB[im:i1, i0:im] @ E[i0:im, j0:j1]) @ LA[j0:j1, j0:j1].T
            rec(im, i1, j0, j1)

    rec(0, m, 0, n)
    return Result(C, Wt, E)


# ---------------------------------------------------------------------------
# Loss and bounds
# ---------------------------------------------------------------------------

def loss(W, V, A, B, scale_mode=SCALE_NONE, scales=None) -> float:
    """tr(B (W - Q) A (W - Q)^T) with Q = s * V, the quadratic form
    ||vec(W - Q)||^2 under the Hessian A (x) B (Proposition 3.1; Appendix A.1
    writes the distortion this way)."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    Q = scale_grid(m, n, scale_mode, scales) * np.asarray(V, dtype=np.float64)
    D = W - Q
    A = sym_from_lower(A)
    B = sym_from_lower(B)
    # trace of the product (B D)(A D^T) without forming it
    return float(np.einsum("ij,ji->", B @ D, A @ D.T))


def loss_from_errors(E: np.ndarray, dA: np.ndarray, dB: np.ndarray) -> float:
    """sum_ij E_ij^2 / (dB_i dA_j)^2. With v - w = Lhat delta and
    Lhat^T H Lhat = diag(d)^-2 (the structure behind Theorem 3.3), this equals
    the loss exactly; d are the un-normalised diagonals of Cholesky(A^-1) and
    Cholesky(B^-1)."""
    E = np.asarray(E, dtype=np.float64)
    return float(np.sum(E ** 2 / (np.asarray(dB)[:, None] * np.asarray(dA)[None, :]) ** 2))


def corollary_3_4_bounds(A, B) -> Tuple[float, float]:
    """Corollary 3.4: loss <= 1/4 sum_ij (R^B_ii)^2 (R^A_jj)^2 <= 1/4 tr(A) tr(B),
    R = RevCholesky. Valid for the unbounded integer alphabet."""
    RA = rev_cholesky(A)
    RB = rev_cholesky(B)
    mid = 0.25 * float(np.sum(np.diag(RB) ** 2) * np.sum(np.diag(RA) ** 2))
    outer = 0.25 * float(np.trace(sym_from_lower(A)) * np.trace(sym_from_lower(B)))
    return mid, outer


# ---------------------------------------------------------------------------
# Checking a solver's codes when floating point may have flipped near-ties
# ---------------------------------------------------------------------------

@dataclass
class ReplayReport:
    inconsistent: int          # entries whose imposed code is not quantize(replayed value)
    max_inconsistent_gap: float  # largest |frac(x/s) - 1/2| over those entries (0 if none)
    Wt: np.ndarray             # replayed pre-rounding values
    gaps: np.ndarray = None    # |frac(x/s) - 1/2| of every inconsistent entry
    E: np.ndarray = None       # replayed errors s*V_given - Wt


def replay(W, LA, LB, alphabet, scale_mode, scales, V_given, leaf: int = 32) -> ReplayReport:
    """Re-run recurrence (2) of Appendix B in float64 with the codes V_given
    imposed (E = s*V_given - replayed value), and report every entry where the
    imposed code differs from what the quantizer would pick at the replayed
    value, together with its distance from the rounding midpoint."""
    res = solve_recursive(W, LA, LB, alphabet, scale_mode, scales, leaf=leaf, forced=V_given)
    m, n = res.Wt.shape
    S = scale_grid(m, n, scale_mode, scales)
    free = quantize(res.Wt, S, alphabet)
    bad = free != np.asarray(V_given, dtype=np.float64)
    gaps = frac_gap(res.Wt[bad] / S[bad])
    gap = float(np.max(gaps)) if gaps.size else 0.0
    return ReplayReport(int(np.count_nonzero(bad)), gap, res.Wt, gaps, res.E)


def frac_gap(x: np.ndarray) -> np.ndarray:
    """|frac(x) - 1/2|: distance of x from the nearest rounding midpoint."""
    x = np.asarray(x, dtype=np.float64)
    return np.abs(x - np.floor(x) - 0.5)
