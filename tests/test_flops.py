"""The closed-form useful-flop count of the band products equals a brute-force
enumeration over entries (Appendix C's two restricted products)."""
import numpy as np
import pytest

import kronecker_factored_gptq_amd as bk
from kronecker_factored_gptq_amd.flops import node_useful_flops, schedule_flops


def brute(m, n, T, k, mid, l):
    ti = np.arange(m) // T
    tj = np.arange(n) // T
    s = ti[:, None] + tj[None, :]
    S1 = (s >= k) & (s < mid)
    S2 = (s >= mid) & (s < l)
    # (p, j) is read by stage 2 iff some q >= j has (p, q) in the target band
    needed = np.flip(np.logical_or.accumulate(np.flip(S2, axis=1), axis=1), axis=1)
    cnt_i_le_p = np.cumsum(S1, axis=0)          # #{i <= p : (i, j) in S1}
    c1 = int(np.sum(np.where(needed, cnt_i_le_p, 0)))
    nz = cnt_i_le_p > 0                          # M[p, j] structurally non-zero
    cnt_j_le_q = np.cumsum(nz, axis=1)           # #{j <= q : M[p, j] != 0}
    c2 = int(np.sum(np.where(S2, cnt_j_le_q, 0)))
    return 2 * c1, 2 * c2


def alg6_nodes(R):
    out = []

    def rec(k, l):
        if l - k == 1:
            return
        mid = (k + l) // 2
        rec(k, mid)
        out.append((k, mid, l))
        rec(mid, l)

    rec(0, R)
    return out


@pytest.mark.parametrize("m,n,T", [(9, 13, 4), (20, 20, 4), (16, 5, 4), (37, 50, 16), (64, 33, 16),
                                   (1, 40, 8), (40, 1, 8), (70, 70, 16)])
def test_closed_form_matches_brute_force(m, n, T):
    R = -(-m // T) + -(-n // T) - 1
    for (k, mid, l) in alg6_nodes(R):
        assert node_useful_flops(m, n, T, k, mid, l) == brute(m, n, T, k, mid, l), (k, mid, l)


def brute_in_block(m, n, T, K0, K1):
    """Entry-level enumeration of a leaf block's in-block updates: inner-sum
    terms (p, i, j) counted once if some target entry reads M[p, j]; outer
    terms (p, q, j) for every target entry and structurally non-zero M[p, j]."""
    ti = np.arange(m) // T
    tj = np.arange(n) // T
    c1 = c2 = 0
    inb = lambda I, J: K0 <= I + J < K1
    for p in range(m):
        P = ti[p]
        for j in range(n):
            J = tj[j]
            # which targets (P, Q) of row-tile P read M[p, j]
            Qs = [Q for Q in range(J, tj[-1] + 1) if inb(P, Q)]
            for i in range(p + 1):
                I = ti[i]
                if not inb(I, J):
                    continue
                if any((I, J) != (P, Q) for Q in Qs):
                    c1 += 1
        for q in range(n):
            Q = tj[q]
            if not inb(P, Q):
                continue
            for j in range(q + 1):
                J = tj[j]
                # M[p, j] for this target has a term from a block tile before (P, Q)
                if any(inb(ti[i], J) and (ti[i], J) != (P, Q) for i in range(p + 1)):
                    c2 += 1
    return 2 * c1, 2 * c2


@pytest.mark.parametrize("m,n,T,K0,K1", [(9, 13, 4, 0, 3), (9, 13, 4, 2, 5), (20, 20, 4, 3, 7),
                                         (16, 5, 4, 1, 4), (13, 30, 4, 4, 9), (30, 13, 4, 0, 12)])
def test_in_block_count_matches_brute_force(m, n, T, K0, K1):
    from kronecker_factored_gptq_amd.flops import in_block_useful_flops
    assert in_block_useful_flops(m, n, T, K0, K1) == brute_in_block(m, n, T, K0, K1)


def test_total_is_of_order_mn_m_plus_n_at_4096():
    """Sum over all nodes at 4096^2 with 16-wide tiles: ~1.8 mn(m+n) flop in
    total (Appendix C's O(mn(m+n))), the bulk of it in the band products (the
    leaves' in-block updates between tiles take a few per cent with 16 tile
    anti-diagonals per leaf block)."""
    ops = bk.solve_schedule(bk.F32, 4096, 4096)
    f = schedule_flops(4096, 4096, 16, ops)
    total = f["in_block"] + f["band"]
    assert 1.6 * 4096 ** 3 * 2 < total < 1.85 * 4096 ** 3 * 2
    assert f["band"] > 0.9 * total
    print(f["band"], f["in_block"])
