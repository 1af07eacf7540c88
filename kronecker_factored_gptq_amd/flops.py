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


def in_block_useful_flops(m: int, n: int, T: int, K0: int, K1: int) -> Tuple[int, int]:
    """(stage-1 flops, stage-2 flops) of the updates between the tiles of one
    leaf block, tile anti-diagonals [K0, K1), as the leaf block computes them
    (left-looking, with each tile row's inner sums carried from tile to tile):
        M[P, J]  = sum_I L^B[P, I] E[I, J]     over block tiles (I, J), I <= P
        W[P, Q] += sum_J M[P, J] L^A[Q, J]^T   for every block tile (P, Q),
    where target (P, Q) takes only errors of the tiles before it
    ((I, J) != (P, Q), I <= P, J <= Q). Every inner-sum term (P, I, J) is
    counted ONCE, whatever number of later tiles reads the carried sum,
    and only if some target reads it; triangular zeros of the diagonal
    tiles and tile padding are not counted (entry granularity)."""
    Mt, Nt = -(-m // T), -(-n // T)
    rows = _tile_sizes(m, T)
    cols = _tile_sizes(n, T)
    s1 = s2 = 0
    for P in range(Mt):
        rp = int(rows[P])
        tri = rp * (rp + 1) // 2
        Qlo, Qhi = max(K0 - P, 0), min(K1 - 1 - P, Nt - 1)
        # stage 1: source tiles (I, J) of the block with I <= P
        for J in range(0, min(K1 - 1, Nt - 1) + 1):
            Ilo, Ihi = max(K0 - J, 0), min(P, K1 - 1 - J, Mt - 1)
            if Ilo > Ihi:
                continue
            cj = int(cols[J])
            for I in range(Ilo, Ihi + 1):
                if I < P:
                    if P + J <= K1 - 1:          # target (P, J) reads it
                        s1 += rp * int(rows[I]) * cj
                elif J + 1 <= Nt - 1 and P + J + 1 <= K1 - 1:  # I == P: targets (P, Q > J)
                    s1 += tri * cj
        # stage 2: targets (P, Q) of the block
        for Q in range(Qlo, Qhi + 1):
            cq = int(cols[Q])
            for J in range(0, Q):
                if P + J >= K0:                  # some (I <= P, J) lies in the block
                    s2 += rp * cq * int(cols[J])
            if P >= 1 and P - 1 + Q >= K0:       # J == Q: sources (I < P, Q)
                s2 += rp * (cq * (cq + 1) // 2)
    return 2 * s1, 2 * s2


def schedule_flops(m: int, n: int, T: int, ops: Iterable[Tuple[int, int, int, int]]
                   ) -> Dict[str, int]:
    """Useful flops of the updates between tiles in a solve schedule: kinds
    2 and 3 are the two band products of an internal node; a leaf block
    (kind 0, tile anti-diagonals [K0, K1)) applies the block's in-block
    updates (``in_block_useful_flops``), reported as "in_block"."""
    out = {"in_block": 0, "band": 0, "band_stage1": 0, "band_stage2": 0, "per_op": []}
    for (kind, k, mid, l) in ops:
        if kind == 0:
            f = sum(in_block_useful_flops(m, n, T, k, mid))
            out["in_block"] += f
            out["per_op"].append(f)
            continue
        f1, f2 = node_useful_flops(m, n, T, k, mid, l)
        if kind == 2:
            out["band"] += f1
            out["band_stage1"] += f1
            out["per_op"].append(f1)
        else:
            out["band"] += f2
            out["band_stage2"] += f2
            out["per_op"].append(f2)
    return out
