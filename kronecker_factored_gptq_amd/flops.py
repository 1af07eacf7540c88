"""Useful-flop count of the solve's internal-node updates (host-side measurement).

At an internal node over tile anti-diagonals [k, l) split at mid, the update
is the pair of restricted band products of "BaKron: Efficient Quantization
with Kronecker-Factored Hessians" (arXiv 2608.06291), Appendix C:
    M[p, j]  = sum_i L^B[p, i] E[i, j]     (i <= p, (i, j) in the source band)
    W[p, q] += sum_j M[p, j] L^A[q, j]     (j <= q, (p, q) in the target band)
Useful work counts one multiply-add (2 flop) per term that is structurally
non-zero at ENTRY granularity: triangular zeros, tile padding, zero tiles
and entries of M that no target reads are not counted. Source band: entries
whose tiles lie on tile anti-diagonals [k, mid); target band: [mid, l).

The count is exact and computed per tile pair in closed form; tests check it
against a brute-force enumeration over entries.
"""
from __future__ import annotations

from typing import Dict, Iterable, Tuple

import numpy as np


def _tile_sizes(d: int, T: int) -> np.ndarray:
    nt = -(-d // T)
    s = np.full(nt, T, dtype=np.int64)
    if nt:
        s[-1] = d - T * (nt - 1)
    return s


def _G(x: np.ndarray, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """sum over rows p = 0..x-1 of #{i in [a, b) : i <= p}."""
    x = x.astype(np.int64)
    w = np.maximum(b - a, 0)
    r1 = np.clip(x - a, 0, None)           # rows p with p+1 > a, up to x
    r1 = np.minimum(r1, w)                  # ... while p+1 <= b
    tri = r1 * (r1 + 1) // 2
    rest = np.clip(x - np.maximum(b, a), 0, None) * w
    return tri + rest


def node_useful_flops(m: int, n: int, T: int, k: int, mid: int, l: int) -> Tuple[int, int]:
    """(stage-1 flops, stage-2 flops) of the node [k, l) split at mid."""
    Mt, Nt = -(-m // T), -(-n // T)
    rows = _tile_sizes(m, T)
    cols = _tile_sizes(n, T)
    J = np.arange(Nt, dtype=np.int64)
    P = np.arange(Mt, dtype=np.int64)
    Ilo = np.maximum(0, k - J)
    Ihi = np.minimum(Mt - 1, mid - 1 - J)
    ne = Ihi >= Ilo
    a = T * Ilo
    b = np.minimum(m, T * (Ihi + 1))
    b = np.where(ne, b, a)

    # stage 1: M tiles (P, J) that some target tile of row-tile P reads
    PP, JJ = np.meshgrid(P, J, indexing="ij")
    needed = np.maximum(JJ, mid - PP) <= np.minimum(Nt - 1, l - 1 - PP)
    x_hi = np.minimum(m, T * (PP + 1))
    x_lo = T * PP
    per_col = _G(x_hi, a[None, :], b[None, :]) - _G(x_lo, a[None, :], b[None, :])
    s1 = int(np.sum(np.where(needed & ne[None, :], per_col * cols[None, :], 0)))

    # stage 2: target tiles (P, Q) on [mid, l)
    QQ = JJ
    tgt = (PP + QQ >= mid) & (PP + QQ <= l - 1)
    # sum over J < Q of cols[J] where ne(J) and Ilo(J) <= P
    ok = ne[None, :] & (Ilo[None, :] <= PP)             # (P, J)
    contrib = np.where(ok, cols[None, :], 0)
    prefix = np.cumsum(contrib, axis=1) - contrib        # exclusive prefix over J
    nq = cols[None, :]
    own = np.where(ok, nq * (nq + 1) // 2, 0)            # J == Q, j <= q within the tile
    per_tile = rows[:, None] * (nq * prefix + own)
    s2 = int(np.sum(np.where(tgt, per_tile, 0)))
    return 2 * s1, 2 * s2


def schedule_flops(m: int, n: int, T: int, ops: Iterable[Tuple[int, int, int, int]]
                   ) -> Dict[str, int]:
    """Useful flops of the updates between tiles in a solve schedule: kinds
    2 and 3 are the two band products of an internal node; a leaf (kind 0)
    of tile anti-diagonal K in a block starting at K0 applies the updates
    from [K0, K) to K, counted as the node [K0, K) -> [K, K+1) ("small").
    Returns totals and per-op values."""
    out = {"small": 0, "band": 0, "band_stage1": 0, "band_stage2": 0, "per_op": []}
    for (kind, k, mid, l) in ops:
        if kind == 0:
            f = sum(node_useful_flops(m, n, T, mid, k, k + 1)) if k > mid else 0
            out["small"] += f
            out["per_op"].append(f)
            continue
        f1, f2 = node_useful_flops(m, n, T, k, mid, l)
        if kind == 1:
            out["small"] += f1 + f2
            out["per_op"].append(f1 + f2)
        elif kind == 2:
            out["band"] += f1
            out["band_stage1"] += f1
            out["per_op"].append(f1)
        else:
            out["band"] += f2
            out["band_stage2"] += f2
            out["per_op"].append(f2)
    return out
