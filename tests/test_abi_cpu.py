"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import kronecker_factored_gptq_amd as bk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bakron.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bakron_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = bk.lib()
    names = declared_functions()
    assert len(names) >= 10
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings_and_version():
    L = bk.lib()
    assert L.bakron_abi_version() == 1
    for st in (0, -1, -2, -3, -4):
        assert L.bakron_status_string(st) != L.bakron_status_string(99)
    assert bk.tile_size(bk.F32) == bk.tile_size(bk.F64) == 16
    assert bk.tile_size(7) == 0


def test_workspace_queries_scale_with_size():
    L = bk.lib()
    for q in (L.bakron_solve_workspace_bytes, L.bakron_factor_workspace_bytes,
              L.bakron_loss_workspace_bytes):
        a = q(bk.F32, 64, 64)
        b = q(bk.F32, 512, 512)
        assert 0 < a < b
        assert q(bk.F64, 512, 512) >= b
        assert q(9, 4, 4) == 0 and q(bk.F32, -1, 4) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def _solve(**kw):
    a = dict(dtype=bk.F32, m=4, n=4, W=FAKE, ldw=4, LA=FAKE, ldla=4, LB=FAKE, ldlb=4, lo=-8, hi=7,
             unb=0, mode=0, scales=None, V=FAKE, ldv=4, Wt=None, ldwt=0, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return bk.lib().bakron_solve(a["dtype"], a["m"], a["n"], a["W"], a["ldw"], a["LA"], a["ldla"],
                                 a["LB"], a["ldlb"], a["lo"], a["hi"], a["unb"], a["mode"],
                                 a["scales"], a["V"], a["ldv"], a["Wt"], a["ldwt"], a["ws"],
                                 a["wsb"], a["stream"])


@pytest.mark.parametrize("bad", [
    dict(dtype=5), dict(m=-1), dict(W=None), dict(LA=None), dict(V=None), dict(ldw=3),
    dict(ldla=2), dict(ldlb=3), dict(ldv=1), dict(lo=3, hi=2), dict(mode=1, scales=None),
    dict(mode=0, scales=FAKE), dict(mode=9), dict(ws=None), dict(wsb=16),
    dict(ws=ctypes.c_void_p(0x1001)), dict(Wt=FAKE, ldwt=2),
])
def test_solve_rejects_bad_arguments(bad):
    assert _solve(**bad) == bk.EINVAL


def test_solve_empty_is_noop():
    assert _solve(m=0, W=None, LA=None, LB=None, V=None, ws=None) == bk.OK
    assert _solve(n=0, W=None, LA=None, LB=None, V=None, ws=None) == bk.OK


def _solve_batched(**kw):
    a = dict(dtype=bk.F32, batch=3, m=4, n=4, W=FAKE, ldw=4, sw=16, LA=FAKE, ldla=4, sla=16,
             LB=FAKE, ldlb=4, slb=16, lo=-8, hi=7, unb=0, mode=0, scales=None, ss=0, V=FAKE,
             ldv=4, sv=16, Wt=None, ldwt=0, swt=0, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return bk.lib().bakron_solve_batched(
        a["dtype"], a["batch"], a["m"], a["n"], a["W"], a["ldw"], a["sw"], a["LA"], a["ldla"],
        a["sla"], a["LB"], a["ldlb"], a["slb"], a["lo"], a["hi"], a["unb"], a["mode"], a["scales"],
        a["ss"], a["V"], a["ldv"], a["sv"], a["Wt"], a["ldwt"], a["swt"], a["ws"], a["wsb"],
        a["stream"])


@pytest.mark.parametrize("bad", [
    dict(dtype=5), dict(batch=-1), dict(batch=65536), dict(m=-1), dict(W=None), dict(LB=None),
    dict(V=None), dict(ldw=3), dict(ldv=3), dict(lo=3, hi=2), dict(mode=1, scales=None),
    dict(mode=0, scales=FAKE), dict(sw=-1), dict(sla=-4), dict(ss=-1, mode=1, scales=FAKE),
    # outputs of different problems would overlap
    dict(sv=15), dict(sv=0), dict(Wt=FAKE, ldwt=4, swt=8),
    dict(ws=None), dict(wsb=16), dict(ws=ctypes.c_void_p(0x1001)),
    # strides whose offsets overflow
    dict(sw=1 << 62),
])
def test_solve_batched_rejects_bad_arguments(bad):
    assert _solve_batched(**bad) == bk.EINVAL


def test_solve_batched_empty_and_workspace():
    assert _solve_batched(batch=0, W=None, LA=None, LB=None, V=None, ws=None) == bk.OK
    assert _solve_batched(m=0, W=None, LA=None, LB=None, V=None, ws=None) == bk.OK
    L = bk.lib()
    one = L.bakron_solve_workspace_bytes(bk.F32, 100, 70)
    assert L.bakron_solve_batched_workspace_bytes(bk.F32, 5, 100, 70) == 5 * one
    assert L.bakron_solve_batched_workspace_bytes(bk.F32, -1, 100, 70) == 0
    assert L.bakron_solve_batched_workspace_bytes(bk.F32, 0, 100, 70) == 0


def _factor_batched(**kw):
    a = dict(dtype=bk.F32, batch=3, m=4, n=4, A=FAKE, lda=4, sa=16, B=FAKE, ldb=4, sb=16,
             LA=FAKE, ldla=4, sla=16, LB=FAKE, ldlb=4, slb=16, dA=None, sda=0, dB=None, sdb=0,
             ws=FAKE, wsb=1 << 40)
    a.update(kw)
    bad = (ctypes.c_int64 * 3)(7, 7, 7)
    rc = bk.lib().bakron_factor_batched(
        a["dtype"], a["batch"], a["m"], a["n"], a["A"], a["lda"], a["sa"], a["B"], a["ldb"], a["sb"],
        a["LA"], a["ldla"], a["sla"], a["LB"], a["ldlb"], a["slb"], a["dA"], a["sda"], a["dB"],
        a["sdb"], a["ws"], a["wsb"], bad, None)
    return rc, tuple(bad)


@pytest.mark.parametrize("bad", [
    dict(dtype=4), dict(batch=-1), dict(batch=32768), dict(m=-2), dict(A=None), dict(LB=None),
    dict(lda=3), dict(ldlb=2), dict(sa=-1), dict(sla=15), dict(slb=0), dict(dA=FAKE, sda=3),
    dict(dB=FAKE, sdb=0), dict(ws=None), dict(wsb=64), dict(ws=ctypes.c_void_p(0x1008)),
    dict(sb=1 << 62),
])
def test_factor_batched_rejects_bad_arguments(bad):
    rc, piv = _factor_batched(**bad)
    assert rc == bk.EINVAL and piv == (-1, -1, -1)


def test_factor_batched_empty_and_workspace():
    assert _factor_batched(batch=0, A=None, B=None, LA=None, LB=None, ws=None)[0] == bk.OK
    assert _factor_batched(m=0, n=0, A=None, B=None, LA=None, LB=None, ws=None)[0] == bk.OK
    L = bk.lib()
    one = L.bakron_factor_workspace_bytes(bk.F32, 100, 70)
    five = L.bakron_factor_batched_workspace_bytes(bk.F32, 5, 100, 70)
    assert L.bakron_factor_batched_workspace_bytes(bk.F32, 1, 100, 70) == one
    assert 4 * one < five <= 5 * one
    assert L.bakron_factor_batched_workspace_bytes(bk.F32, -1, 100, 70) == 0


@pytest.mark.parametrize("bad", [
    dict(dtype=2), dict(N=-1), dict(d=-1), dict(X=None), dict(ldx=3), dict(G=None), dict(ldg=3),
    dict(damp=-0.5), dict(damp=float("nan")),
])
def test_gram_rejects_bad_arguments(bad):
    a = dict(dtype=bk.F32, N=5, d=4, X=FAKE, ldx=4, w=None, damp=0.0, G=FAKE, ldg=4)
    a.update(bad)
    L = bk.lib()
    assert L.bakron_gram(a["dtype"], a["N"], a["d"], a["X"], a["ldx"], a["w"], a["damp"], a["G"],
                         a["ldg"], None) == bk.EINVAL
    assert L.bakron_gram(bk.F32, 5, 0, None, 0, None, 0.0, None, 0, None) == bk.OK
    # G overlapping X (in place, or the tail of X) is rejected
    assert L.bakron_gram(bk.F32, 5, 4, FAKE, 4, None, 0.0, FAKE, 4, None) == bk.EINVAL
    assert L.bakron_gram(bk.F32, 5, 4, FAKE, 4, None, 0.0, ctypes.c_void_p(0x1000 + 4 * 19), 4,
                         None) == bk.EINVAL
    assert L.bakron_sample_sqnorms(bk.F32, 5, 4, FAKE, 3, FAKE, None) == bk.EINVAL
    assert L.bakron_sample_sqnorms(bk.F32, 5, 4, FAKE, 4, None, None) == bk.EINVAL
    assert L.bakron_sample_sqnorms(bk.F32, 0, 4, None, 4, None, None) == bk.OK


@pytest.mark.parametrize("bad", [
    dict(dtype=9), dict(batch=-1), dict(batch=65536), dict(W=None), dict(V=None), dict(ldw=3),
    dict(ldb=3), dict(mode=1, scales=None), dict(mode=0, scales=FAKE), dict(mode=5),
    dict(sw=-1), dict(sb=-2), dict(loss=None), dict(ws=None), dict(wsb=32),
    dict(ws=ctypes.c_void_p(0x1004)), dict(sa=1 << 62),
])
def test_loss_batched_rejects_bad_arguments(bad):
    a = dict(dtype=bk.F32, batch=3, m=4, n=4, W=FAKE, ldw=4, sw=16, V=FAKE, ldv=4, sv=16, mode=0,
             scales=None, ss=0, A=FAKE, lda=4, sa=16, B=FAKE, ldb=4, sb=16, loss=FAKE, ws=FAKE,
             wsb=1 << 40)
    a.update(bad)
    rc = bk.lib().bakron_loss_batched(a["dtype"], a["batch"], a["m"], a["n"], a["W"], a["ldw"],
                                      a["sw"], a["V"], a["ldv"], a["sv"], a["mode"], a["scales"],
                                      a["ss"], a["A"], a["lda"], a["sa"], a["B"], a["ldb"], a["sb"],
                                      a["loss"], a["ws"], a["wsb"], None)
    assert rc == bk.EINVAL
    L = bk.lib()
    assert L.bakron_loss_batched_workspace_bytes(bk.F32, 3, 40, 50) == \
        3 * L.bakron_loss_workspace_bytes(bk.F32, 40, 50)


def test_factor_and_loss_reject_bad_arguments():
    L = bk.lib()
    bad = (ctypes.c_int64 * 2)(7, 7)
    rc = L.bakron_factor(bk.F32, 4, 4, None, 4, FAKE, 4, FAKE, 4, FAKE, 4, None, None, FAKE,
                         1 << 40, bad, None)
    assert rc == bk.EINVAL and tuple(bad) == (-1, -1)
    rc = L.bakron_factor(bk.F32, 4, 4, FAKE, 3, FAKE, 4, FAKE, 4, FAKE, 4, None, None, FAKE,
                         1 << 40, None, None)
    assert rc == bk.EINVAL
    rc = L.bakron_factor(bk.F32, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, FAKE, 4, None, None, FAKE, 8,
                         None, None)
    assert rc == bk.EINVAL
    rc = L.bakron_loss(bk.F32, 4, 4, FAKE, 4, FAKE, 4, 0, None, FAKE, 4, FAKE, 4, None, FAKE,
                       1 << 40, None)
    assert rc == bk.EINVAL
    rc = L.bakron_loss(bk.F32, 4, 4, FAKE, 4, FAKE, 4, 2, None, FAKE, 4, FAKE, 4, FAKE, FAKE,
                       1 << 40, None)
    assert rc == bk.EINVAL
    assert L.bakron_row_scales(bk.F32, 4, 4, FAKE, 4, 0, FAKE, None) == bk.EINVAL
    assert L.bakron_row_scales(bk.F32, 4, 4, FAKE, 3, 7, FAKE, None) == bk.EINVAL


@pytest.mark.parametrize("bad", [
    dict(dtype=3), dict(m=-1), dict(hi=0), dict(lo=5, hi=4), dict(grid=-1), dict(grid=1025),
    dict(shrink=-0.1), dict(shrink=1.0), dict(shrink=float("nan")), dict(W=None), dict(ldw=3),
    dict(s=None),
])
def test_row_scales_mse_rejects_bad_arguments(bad):
    a = dict(dtype=bk.F32, m=4, n=4, W=FAKE, ldw=4, lo=-8, hi=7, grid=100, shrink=0.5, s=FAKE)
    a.update(bad)
    L = bk.lib()
    rc = L.bakron_row_scales_mse(a["dtype"], a["m"], a["n"], a["W"], a["ldw"], a["lo"], a["hi"],
                                 a["grid"], a["shrink"], a["s"], None)
    assert rc == bk.EINVAL
    assert L.bakron_row_scales_mse(bk.F32, 0, 4, None, 4, -8, 7, 100, 0.5, None, None) == bk.OK


def _closed_form_leaves(m, n, T=16):
    return -(-m // T) + -(-n // T) - 1


@pytest.mark.parametrize("m,n", [(1, 1), (16, 16), (17, 5), (64, 64), (200, 300), (512, 512),
                                 (4096, 4096), (14336, 4096), (4096, 14336), (1024, 2048)])
def test_schedule_is_algorithm_6_over_blocks_of_tile_antidiagonals(m, n):
    """Table 1 "Steps" for BaKron: the tile anti-diagonals 0 .. R-1 in order,
    in leaf blocks of G (G read from the first block); Algorithm 6's
    recursion over the blocks, each internal node splitting block range
    [kb, lb) at floor((kb+lb)/2) and running after the leaf block left of
    its midpoint and before the one right of it."""
    ops = bk.solve_schedule(bk.F32, m, n)
    R = _closed_form_leaves(m, n)
    leaves = [(a, b) for (kind, a, b, c) in ops if kind == 0]
    BLOCK = leaves[0][1] - leaves[0][0] if len(leaves) > 1 else R + 1  # one block: any G >= R
    nblocks = -(-R // BLOCK)
    assert leaves == [(i * BLOCK, min((i + 1) * BLOCK, R)) for i in range(nblocks)]
    nodes = [(a, b, c) for (kind, a, b, c) in ops if kind == 2]
    assert len(nodes) == nblocks - 1
    assert sorted(mid for (_, mid, _) in nodes) == [BLOCK * i for i in range(1, nblocks)]
    for (k, mid, l) in nodes:
        kb, lb = k // BLOCK, -(-l // BLOCK)
        assert k % BLOCK == 0 and mid == BLOCK * ((kb + lb) // 2) and k < mid < l <= R
    kinds = [op[0] for op in ops]
    assert set(kinds) <= {0, 2, 3}
    for i, kd in enumerate(kinds):
        if kd == 2:
            assert kinds[i + 1] == 3 and ops[i][1:] == ops[i + 1][1:]
    pos = {a: i for i, (kind, a, _, _) in enumerate(ops) if kind == 0}
    end = {b: i for i, (kind, _, b, _) in enumerate(ops) if kind == 0}
    for i, (kind, k, mid, l) in enumerate(ops):
        if kind in (2, 3):
            assert end[mid] < i < pos[mid]


def _noalloc(**kw):
    a = dict(dtype=bk.F32, m=4, n=4, W=FAKE, ldw=4, LA=FAKE, ldla=4, LB=FAKE, ldlb=4, lo=-8, hi=7,
             unb=0, mode=0, scales=None, V=FAKE, ldv=4, Wt=None, ldwt=0, stream=None)
    a.update(kw)
    return bk.lib().bakron_solve_noalloc(a["dtype"], a["m"], a["n"], a["W"], a["ldw"], a["LA"],
                                         a["ldla"], a["LB"], a["ldlb"], a["lo"], a["hi"], a["unb"],
                                         a["mode"], a["scales"], a["V"], a["ldv"], a["Wt"],
                                         a["ldwt"], a["stream"])


@pytest.mark.parametrize("dtype,m,n", [
    (bk.F32, 2600, 2600),   # a float32 square just over 96 MiB of workspace
    (bk.F32, 4096, 4096),
    (bk.F64, 2048, 2048),
    (bk.F64, 1 << 20, 1),
])
def test_noalloc_rejects_sizes_beyond_its_scratch(dtype, m, n):
    """The size check runs before any HIP call (so it is testable here)."""
    L = bk.lib()
    assert L.bakron_solve_workspace_bytes(dtype, m, n) > bk.NOALLOC_SCRATCH_BYTES
    assert _noalloc(dtype=dtype, m=m, n=n, ldw=n, ldla=n, ldlb=m, ldv=n) == bk.EINVAL


def test_noalloc_limit_admits_the_stated_shapes():
    L = bk.lib()
    assert L.bakron_solve_workspace_bytes(bk.F32, 2048, 2048) <= bk.NOALLOC_SCRATCH_BYTES
    assert L.bakron_solve_workspace_bytes(bk.F64, 1024, 2048) <= bk.NOALLOC_SCRATCH_BYTES


def test_noalloc_argument_errors_and_empty():
    assert _noalloc(dtype=5) == bk.EINVAL
    assert _noalloc(m=-1) == bk.EINVAL
    assert _noalloc(m=0, W=None, LA=None, LB=None, V=None) == bk.OK
    assert _noalloc(n=0, W=None, LA=None, LB=None, V=None) == bk.OK


def _antidiag(**kw):
    a = dict(dtype=bk.F32, m=4, n=4, W=FAKE, ldw=4, LA=FAKE, ldla=4, LB=FAKE, ldlb=4, lo=-8, hi=7,
             unb=0, mode=0, scales=None, V=FAKE, ldv=4, Wt=None, ldwt=0, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return bk.lib().bakron_solve_antidiag(a["dtype"], a["m"], a["n"], a["W"], a["ldw"], a["LA"],
                                          a["ldla"], a["LB"], a["ldlb"], a["lo"], a["hi"], a["unb"],
                                          a["mode"], a["scales"], a["V"], a["ldv"], a["Wt"],
                                          a["ldwt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("bad", [
    dict(dtype=5), dict(m=-1), dict(W=None), dict(LA=None), dict(V=None), dict(ldw=3),
    dict(ldla=2), dict(ldlb=3), dict(ldv=1), dict(lo=3, hi=2), dict(mode=1, scales=None),
    dict(mode=0, scales=FAKE), dict(mode=9), dict(ws=None), dict(wsb=16),
    dict(ws=ctypes.c_void_p(0x1001)), dict(Wt=FAKE, ldwt=2),
])
def test_antidiag_rejects_bad_arguments(bad):
    assert _antidiag(**bad) == bk.EINVAL


def test_antidiag_empty_is_noop_and_workspace_grows():
    assert _antidiag(m=0, W=None, LA=None, LB=None, V=None, ws=None) == bk.OK
    L = bk.lib()
    assert 0 < L.bakron_solve_antidiag_workspace_bytes(bk.F32, 64, 64) < \
        L.bakron_solve_antidiag_workspace_bytes(bk.F32, 512, 512) < \
        L.bakron_solve_antidiag_workspace_bytes(bk.F64, 512, 512)


def test_blockdiag_queries_and_argument_errors():
    L = bk.lib()
    # heads must divide m and be at least 1
    for heads, m in ((0, 8), (3, 8), (-1, 8)):
        assert L.bakron_factor_blockdiag_workspace_bytes(bk.F32, heads, m, 4) == 0
        assert L.bakron_solve_blockdiag_workspace_bytes(bk.F32, heads, m, 4) == 0
        assert L.bakron_loss_blockdiag_workspace_bytes(bk.F32, heads, m, 4) == 0
    assert L.bakron_solve_blockdiag_workspace_bytes(bk.F32, 4, 64, 32) == \
        L.bakron_solve_batched_workspace_bytes(bk.F32, 4, 16, 32)
    bad = (bk._i64 * 3)(0, 0, 0)
    # factor: heads not dividing m, then a block stride that overlaps the outputs
    assert L.bakron_factor_blockdiag(bk.F32, 3, 8, 4, FAKE, 4, FAKE, 8, 64, FAKE, 4, FAKE, 8, 64,
                                     None, None, FAKE, 1 << 40, bad, None) == bk.EINVAL
    assert tuple(bad) == (-1, -1, -1)
    assert L.bakron_factor_blockdiag(bk.F32, 2, 8, 4, FAKE, 4, FAKE, 4, 16, FAKE, 4, FAKE, 4, 4,
                                     None, None, FAKE, 1 << 40, bad, None) == bk.EINVAL
    # solve: heads not dividing m; empty problem
    assert L.bakron_solve_blockdiag(bk.F32, 3, 8, 4, FAKE, 4, FAKE, 4, FAKE, 2, 4, -8, 7, 0, 0,
                                    None, FAKE, 4, None, 0, FAKE, 1 << 40, None) == bk.EINVAL
    assert L.bakron_solve_blockdiag(bk.F32, 2, 8, 0, None, 0, None, 0, None, 4, 16, -8, 7, 0, 0,
                                    None, None, 0, None, 0, None, 0, None) == bk.OK
    # loss: no output pointer, then a bad scale mode
    assert L.bakron_loss_blockdiag(bk.F32, 2, 8, 4, FAKE, 4, FAKE, 4, 0, None, FAKE, 4, FAKE, 4, 16,
                                   None, FAKE, 1 << 40, None) == bk.EINVAL
    assert L.bakron_loss_blockdiag(bk.F32, 2, 8, 4, FAKE, 4, FAKE, 4, 7, None, FAKE, 4, FAKE, 4, 16,
                                   FAKE, FAKE, 1 << 40, None) == bk.EINVAL


def test_solve_status_arguments_and_wait_hook():
    L = bk.lib()
    # bad arguments are refused before any HIP call; empty problems are OK
    assert L.bakron_solve_status(7, 1, 4, 4, FAKE, 1 << 20, None) == bk.EINVAL
    assert L.bakron_solve_status(bk.F32, -1, 4, 4, FAKE, 1 << 20, None) == bk.EINVAL
    assert L.bakron_solve_status(bk.F32, 1, -4, 4, FAKE, 1 << 20, None) == bk.EINVAL
    assert L.bakron_solve_status(bk.F32, 0, 4, 4, FAKE, 0, None) == bk.OK
    assert L.bakron_solve_status(bk.F32, 1, 0, 4, FAKE, 0, None) == bk.OK
    # a workspace smaller than the batch's solve workspace
    need = L.bakron_solve_batched_workspace_bytes(bk.F32, 3, 40, 50)
    assert L.bakron_solve_status(bk.F32, 3, 40, 50, FAKE, need - 1, None) == bk.EINVAL
    # the no-allocation scratch holds one problem of at most its size
    assert L.bakron_solve_status(bk.F32, 2, 40, 50, None, 0, None) == bk.EINVAL
    assert L.bakron_solve_status(bk.F32, 1, 4096, 4096, None, 0, None) == bk.EINVAL
    # the poll bound hook: set, read back, restore the default
    prev = bk.debug_set_wait_polls(0)
    assert bk.debug_set_wait_polls(5) == 0
    assert bk.debug_set_wait_polls(-1) == 5
    assert bk.debug_set_wait_polls(prev) == prev
