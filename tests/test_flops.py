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


def test_total_is_of_order_mn_m_plus_n_at_4096():
    """Sum over all nodes at 4096^2 with 16-wide tiles: ~1.8 mn(m+n) flop in
    total (Appendix C's O(mn(m+n))), the bulk of it in the band products (the
    leaves' in-block updates take the rest: 7 % with 12 tile anti-diagonals
    per leaf block)."""
    ops = bk.solve_schedule(bk.F32, 4096, 4096)
    f = schedule_flops(4096, 4096, 16, ops)
    total = f["small"] + f["band"]
    assert 1.6 * 4096 ** 3 * 2 < total < 1.85 * 4096 ** 3 * 2
    assert f["band"] > 0.9 * total
