"""MI355X-native BaKron solver.

A thin Python binding over the C ABI of ``libbakron.so`` (include/bakron.h):
argument marshalling only. PyTorch supplies device memory and streams; every
step of the computation runs in the library's HIP kernels. The binding fails
loudly when the library is missing; there is no fallback path.

BaKron ("BaKron: Efficient Quantization with Kronecker-Factored Hessians",
arXiv 2608.06291) quantises W (m x n) with GPTQ on vec(W) under the Hessian
A (x) B, A n x n (input side) and B m x m (output side).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

__all__ = ["F32", "F64", "SCALE_NONE", "SCALE_ROW", "SCALE_COL", "BakronError", "lib", "factor",
           "factor_batched",
           "solve", "solve_antidiag", "solve_noalloc", "factor_blockdiag", "solve_blockdiag",
           "loss_blockdiag", "solve_batched", "loss", "loss_batched", "row_scales", "row_scales_mse", "gram",
           "sample_sqnorms", "kfac_factors", "shampoo_factors", "solve_schedule", "tile_size", "workspace_bytes"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libbakron.so")

F32, F64 = 0, 1
SCALE_NONE, SCALE_ROW, SCALE_COL = 0, 1, 2
OK, EINVAL, ENOTSPD, EHIP, EWAIT = 0, -1, -2, -3, -4


class BakronError(RuntimeError):
    def __init__(self, status: int, what: str, bad_pivot: Optional[Tuple[int, int]] = None):
        self.status = status
        self.bad_pivot = bad_pivot
        msg = f"{what}: {_status_string(status)} (status {status})"
        if bad_pivot is not None and bad_pivot[0] >= 0:
            side = "A" if bad_pivot[0] == 0 else "B"
            msg += f"; failing pivot {bad_pivot[1]} of the reversed Cholesky of {side}"
        super().__init__(msg)


_lib = None
_vp, _i64, _i32, _sz, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_int


def lib() -> ctypes.CDLL:
    """Load libbakron.so (built by __graft_entry__.build() or
    ``python -m kronecker_factored_gptq_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(f"{LIB_PATH} is not built; run `python -m kronecker_factored_gptq_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.bakron_status_string.argtypes = [_int]
    L.bakron_status_string.restype = ctypes.c_char_p
    L.bakron_abi_version.argtypes = []
    L.bakron_abi_version.restype = _int
    L.bakron_tile_size.argtypes = [_int]
    L.bakron_tile_size.restype = _int
    for name in ("bakron_factor_workspace_bytes", "bakron_solve_workspace_bytes",
                 "bakron_loss_workspace_bytes"):
        f = getattr(L, name)
        f.argtypes = [_int, _i64, _i64]
        f.restype = _sz
    L.bakron_factor.argtypes = [_int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                _vp, _vp, _vp, _sz, ctypes.POINTER(_i64), _vp]
    L.bakron_factor.restype = _int
    L.bakron_solve.argtypes = [_int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i32, _i32, _i32,
                               _int, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp]
    L.bakron_solve.restype = _int
    for name in ("bakron_factor_blockdiag_workspace_bytes", "bakron_solve_blockdiag_workspace_bytes",
                 "bakron_loss_blockdiag_workspace_bytes"):
        f = getattr(L, name)
        f.argtypes = [_int, _i64, _i64, _i64]
        f.restype = _sz
    L.bakron_factor_blockdiag.argtypes = [_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp,
                                          _i64, _vp, _i64, _i64, _vp, _vp, _vp, _sz,
                                          ctypes.POINTER(_i64), _vp]
    L.bakron_factor_blockdiag.restype = _int
    L.bakron_solve_blockdiag.argtypes = [_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                         _i64, _i32, _i32, _i32, _int, _vp, _vp, _i64, _vp, _i64,
                                         _vp, _sz, _vp]
    L.bakron_solve_blockdiag.restype = _int
    L.bakron_loss_blockdiag.argtypes = [_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _int, _vp,
                                        _vp, _i64, _vp, _i64, _i64, _vp, _vp, _sz, _vp]
    L.bakron_loss_blockdiag.restype = _int
    L.bakron_solve_antidiag_workspace_bytes.argtypes = [_int, _i64, _i64]
    L.bakron_solve_antidiag_workspace_bytes.restype = _sz
    L.bakron_solve_antidiag.argtypes = L.bakron_solve.argtypes
    L.bakron_solve_antidiag.restype = _int
    L.bakron_solve_noalloc.argtypes = [_int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i32,
                                       _i32, _i32, _int, _vp, _vp, _i64, _vp, _i64, _vp]
    L.bakron_solve_noalloc.restype = _int
    L.bakron_solve_timed.argtypes = L.bakron_solve.argtypes + [_vp, _i64]
    L.bakron_solve_timed.restype = _int
    L.bakron_solve_status.argtypes = [_int, _i64, _i64, _i64, _vp, _sz, _vp]
    L.bakron_solve_status.restype = _int
    L.bakron_debug_set_wait_polls.argtypes = [_i32]
    L.bakron_debug_set_wait_polls.restype = _i32
    L.bakron_solve_schedule.argtypes = [_int, _i64, _i64, _vp, _i64]
    L.bakron_solve_schedule.restype = _i64
    L.bakron_factor_batched_workspace_bytes.argtypes = [_int, _i64, _i64, _i64]
    L.bakron_factor_batched_workspace_bytes.restype = _sz
    L.bakron_factor_batched.argtypes = [_int, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                        _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64,
                                        _vp, _sz, ctypes.POINTER(_i64), _vp]
    L.bakron_factor_batched.restype = _int
    L.bakron_solve_batched_workspace_bytes.argtypes = [_int, _i64, _i64, _i64]
    L.bakron_solve_batched_workspace_bytes.restype = _sz
    L.bakron_solve_batched.argtypes = [_int, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                       _vp, _i64, _i64, _i32, _i32, _i32, _int, _vp, _i64,
                                       _vp, _i64, _i64, _vp, _i64, _i64, _vp, _sz, _vp]
    L.bakron_solve_batched.restype = _int
    L.bakron_loss.argtypes = [_int, _i64, _i64, _vp, _i64, _vp, _i64, _int, _vp, _vp, _i64, _vp,
                              _i64, _vp, _vp, _sz, _vp]
    L.bakron_loss.restype = _int
    L.bakron_loss_batched_workspace_bytes.argtypes = [_int, _i64, _i64, _i64]
    L.bakron_loss_batched_workspace_bytes.restype = _sz
    L.bakron_loss_batched.argtypes = [_int, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                      _int, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp,
                                      _sz, _vp]
    L.bakron_loss_batched.restype = _int
    L.bakron_row_scales.argtypes = [_int, _i64, _i64, _vp, _i64, _i32, _vp, _vp]
    L.bakron_row_scales.restype = _int
    L.bakron_row_scales_mse.argtypes = [_int, _i64, _i64, _vp, _i64, _i32, _i32, _i32,
                                        ctypes.c_double, _vp, _vp]
    L.bakron_row_scales_mse.restype = _int
    L.bakron_gram.argtypes = [_int, _i64, _i64, _vp, _i64, _vp, ctypes.c_double, _vp, _i64, _vp]
    L.bakron_gram.restype = _int
    L.bakron_sample_sqnorms.argtypes = [_int, _i64, _i64, _vp, _i64, _vp, _vp]
    L.bakron_sample_sqnorms.restype = _int
    _lib = L
    return L


def _status_string(status: int) -> str:
    try:
        return lib().bakron_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - library missing
        return "unknown"


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float64:
        return F64
    raise TypeError(f"expected float32 or float64, got {t.dtype}")


def _tdt(code: int) -> torch.dtype:
    return torch.float32 if code == F32 else torch.float64


def _ld(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    return max(int(t.stride(0)), int(t.size(1)), 1)


def _check_out(t: torch.Tensor, shape, dtype: torch.dtype, name: str) -> None:
    """A caller-supplied output must have exactly the shape and element type
    the kernels write, with unit column stride (the C ABI only sees its
    pointer and leading dimension)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() == 2 and t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    if t.dim() == 2 and t.size(0) > 1 and t.stride(0) < t.size(1):
        raise ValueError(f"{name} rows overlap (leading dimension below the row length)")


def _check_operand(t: torch.Tensor, shape, dtype: torch.dtype, name: str) -> None:
    """An input read by the kernels: exact shape and element type."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_device(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _workspace(nbytes: int, dev, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


def tile_size(dtype: int = F32) -> int:
    return int(lib().bakron_tile_size(int(dtype)))


def workspace_bytes(kind: str, dtype: int, m: int, n: int) -> int:
    f = {"factor": lib().bakron_factor_workspace_bytes, "solve": lib().bakron_solve_workspace_bytes,
         "loss": lib().bakron_loss_workspace_bytes}[kind]
    return int(f(int(dtype), int(m), int(n)))


def factor(A: torch.Tensor, B: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
           workspace: Optional[torch.Tensor] = None):
    """L^A = Cholesky(A^-1), L^B = Cholesky(B^-1), columns normalised by their
    diagonals (§3.2 Algorithm 2), plus the diagonals dA, dB. Synchronous.
    Raises BakronError(ENOTSPD) for a non-positive-definite input."""
    dev = _check_device(A, B)
    code = _dt(A)
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same dtype")
    if out_dtype is not None and out_dtype != A.dtype:
        raise TypeError("out_dtype must equal the input dtype")
    n, m = A.size(0), B.size(0)
    if A.shape != (n, n) or B.shape != (m, m):
        raise ValueError("A and B must be square")
    LA = torch.empty((n, n), dtype=A.dtype, device=dev)
    LB = torch.empty((m, m), dtype=A.dtype, device=dev)
    dA = torch.empty(n, dtype=A.dtype, device=dev)
    dB = torch.empty(m, dtype=A.dtype, device=dev)
    L = lib()
    nbytes = L.bakron_factor_workspace_bytes(code, m, n)
    ws = _workspace(nbytes, dev, workspace)
    bad = (_i64 * 2)(-1, -1)
    with torch.cuda.device(dev):
        rc = L.bakron_factor(code, m, n, _p(A), _ld(A, "A"), _p(B), _ld(B, "B"), _p(LA), n,
                             _p(LB), m, _p(dA), _p(dB), _p(ws), ws.numel(), bad, _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_factor", (int(bad[0]), int(bad[1])))
    return LA, LB, dA, dB


def factor_batched(A: torch.Tensor, B: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """bakron_factor on a batch of pairs of the same orders in the same
    launches. A is (batch, n, n), B (batch, m, m). Returns LA (batch, n, n),
    LB (batch, m, m), dA (batch, n), dB (batch, m); each pair's result is
    bit-identical to ``factor``. Synchronous. Raises BakronError(ENOTSPD)
    with ``bad_pivot`` = (pair, side, index)."""
    dev = _check_device(A, B, workspace)
    code = _dt(A)
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same dtype")
    if A.dim() != 3 or B.dim() != 3 or A.size(0) != B.size(0):
        raise ValueError("A must be (batch, n, n) and B (batch, m, m)")
    batch, n, m = A.size(0), A.size(1), B.size(1)
    pa, lda, sa = _batch_operand(A, n, n, batch, "A")
    pb, ldb, sb = _batch_operand(B, m, m, batch, "B")
    LA = torch.empty((batch, n, n), dtype=A.dtype, device=dev)
    LB = torch.empty((batch, m, m), dtype=A.dtype, device=dev)
    dA = torch.empty((batch, n), dtype=A.dtype, device=dev)
    dB = torch.empty((batch, m), dtype=A.dtype, device=dev)
    L = lib()
    ws = _workspace(L.bakron_factor_batched_workspace_bytes(code, batch, m, n), dev, workspace)
    bad = (_i64 * 3)(-1, -1, -1)
    with torch.cuda.device(dev):
        rc = L.bakron_factor_batched(code, batch, m, n, pa, lda, sa, pb, ldb, sb, _p(LA), max(n, 1),
                                     n * n, _p(LB), max(m, 1), m * m, _p(dA), n, _p(dB), m, _p(ws),
                                     ws.numel() * ws.element_size(), bad, _stream(dev))
    if rc != OK:
        err = BakronError(rc, "bakron_factor_batched", (int(bad[1]), int(bad[2])))
        err.bad_pivot = (int(bad[0]), int(bad[1]), int(bad[2]))
        raise err
    return LA, LB, dA, dB


AlphabetLike = Union[Sequence[int], Tuple[int, int, int]]


def _scale_mode(scales: Optional[torch.Tensor], m: int, n: int, scale_mode: Optional[int]) -> int:
    if scales is None:
        if scale_mode not in (None, SCALE_NONE):
            raise ValueError("scales required for this scale_mode")
        return SCALE_NONE
    if scale_mode is None:
        if scales.numel() == m:
            return SCALE_ROW
        if scales.numel() == n:
            return SCALE_COL
        raise ValueError("scales must have length m (rows) or n (columns)")
    want = m if scale_mode == SCALE_ROW else n
    if scale_mode not in (SCALE_ROW, SCALE_COL) or scales.numel() != want:
        raise ValueError("scales do not match scale_mode")
    return scale_mode


def solve(W: torch.Tensor, LA: torch.Tensor, LB: torch.Tensor, alphabet: AlphabetLike = (0, 0, 1),
          scales: Optional[torch.Tensor] = None, scale_mode: Optional[int] = None,
          return_wt: bool = False, workspace: Optional[torch.Tensor] = None,
          out: Optional[torch.Tensor] = None, op_ms: Optional[ctypes.Array] = None,
          check: bool = False):
    """BaKron solve (§3.5 Algorithm 6 on a tiling of W). Returns int32 codes V
    (m x n), and with ``return_wt`` also the value each entry had when it was
    rounded. Asynchronous on the current stream, except with ``op_ms`` (a
    ctypes double array, one slot per schedule record: every leaf-block and
    band-product launch is timed with HIP events and the call waits for
    them) or ``check`` (waits, then raises BakronError(EWAIT) if a leaf
    block's bounded wait gave up)."""
    dev = _check_device(W, LA, LB, scales, workspace, out)
    code = _dt(W)
    m, n = W.shape
    if LA.shape != (n, n) or LB.shape != (m, m) or LA.dtype != W.dtype or LB.dtype != W.dtype:
        raise ValueError("LA must be n x n and LB m x m, same dtype as W")
    lo, hi, unb = (int(alphabet[0]), int(alphabet[1]), int(bool(alphabet[2])))
    mode = _scale_mode(scales, m, n, scale_mode)
    if scales is not None:
        if scales.dtype != W.dtype or not scales.is_contiguous():
            raise ValueError("scales must be contiguous with W's dtype")
    if out is not None:
        _check_out(out, (m, n), torch.int32, "out")
    V = out if out is not None else torch.empty((m, n), dtype=torch.int32, device=dev)
    Wt = torch.empty((m, n), dtype=W.dtype, device=dev) if return_wt else None
    L = lib()
    ws = _workspace(L.bakron_solve_workspace_bytes(code, m, n), dev, workspace)
    args = (code, m, n, _p(W), _ld(W, "W"), _p(LA), _ld(LA, "LA"), _p(LB), _ld(LB, "LB"), lo, hi,
            unb, mode, _p(scales), _p(V), _ld(V, "V"), _p(Wt),
            _ld(Wt, "Wt") if Wt is not None else 0, _p(ws), ws.numel() * ws.element_size(),
            _stream(dev))
    with torch.cuda.device(dev):
        if op_ms is None:
            rc = L.bakron_solve(*args)
        else:
            rc = L.bakron_solve_timed(*args, ctypes.cast(op_ms, ctypes.c_void_p), len(op_ms))
    if rc == OK and check:
        rc = L.bakron_solve_status(code, 1, m, n, _p(ws), ws.numel() * ws.element_size(),
                                   _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_solve")
    return (V, Wt) if return_wt else V


def solve_antidiag(W: torch.Tensor, LA: torch.Tensor, LB: torch.Tensor,
                   alphabet: AlphabetLike = (0, 0, 1), scales: Optional[torch.Tensor] = None,
                   scale_mode: Optional[int] = None, return_wt: bool = False,
                   workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """BaKron-antidiagonal (§3.3 Algorithm 3 on the whole matrix, one launch
    per anti-diagonal): the same codes as ``solve`` (Theorem 3.2) with
    O(m^2 n^2) work, the paper's point of comparison. Arguments and results
    as for ``solve``. Asynchronous on the current stream."""
    dev = _check_device(W, LA, LB, scales, workspace, out)
    code = _dt(W)
    m, n = W.shape
    if LA.shape != (n, n) or LB.shape != (m, m) or LA.dtype != W.dtype or LB.dtype != W.dtype:
        raise ValueError("LA must be n x n and LB m x m, same dtype as W")
    lo, hi, unb = (int(alphabet[0]), int(alphabet[1]), int(bool(alphabet[2])))
    mode = _scale_mode(scales, m, n, scale_mode)
    if scales is not None and (scales.dtype != W.dtype or not scales.is_contiguous()):
        raise ValueError("scales must be contiguous with W's dtype")
    if out is not None:
        _check_out(out, (m, n), torch.int32, "out")
    V = out if out is not None else torch.empty((m, n), dtype=torch.int32, device=dev)
    Wt = torch.empty((m, n), dtype=W.dtype, device=dev) if return_wt else None
    L = lib()
    ws = _workspace(L.bakron_solve_antidiag_workspace_bytes(code, m, n), dev, workspace)
    with torch.cuda.device(dev):
        rc = L.bakron_solve_antidiag(code, m, n, _p(W), _ld(W, "W"), _p(LA), _ld(LA, "LA"), _p(LB),
                                     _ld(LB, "LB"), lo, hi, unb, mode, _p(scales), _p(V),
                                     _ld(V, "V"), _p(Wt), _ld(Wt, "Wt") if Wt is not None else 0,
                                     _p(ws), ws.numel() * ws.element_size(), _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_solve_antidiag")
    return (V, Wt) if return_wt else V


def _blocks(t: torch.Tensor, heads: int, b: int, name: str):
    """(pointer, ld, stride) of h square blocks given as a (heads, b, b) tensor."""
    if t.dim() != 3 or t.shape != (heads, b, b):
        raise ValueError(f"{name} must be ({heads}, {b}, {b})")
    if b > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    ld = max(int(t.stride(1)), b, 1)
    return _p(t), ld, int(t.stride(0)) if heads > 1 else 0


def factor_blockdiag(A: torch.Tensor, Bblocks: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """L^A of A (n x n) and the normalised Cholesky(B_h^-1) of every block of
    a block-diagonal output factor B = blockdiag(Bblocks[h]) (Bblocks is
    (heads, b, b)). Returns LA (n x n), LB blocks (heads, b, b), dA (n),
    dB (heads * b). Synchronous. BakronError.bad_pivot = (side, block, index)."""
    dev = _check_device(A, Bblocks, workspace)
    code = _dt(A)
    if Bblocks.dtype != A.dtype:
        raise TypeError("A and the B blocks must have the same dtype")
    n = A.size(0)
    if A.shape != (n, n) or Bblocks.dim() != 3:
        raise ValueError("A must be n x n and Bblocks (heads, b, b)")
    heads, b = Bblocks.size(0), Bblocks.size(1)
    pb, ldb, sb = _blocks(Bblocks, heads, b, "Bblocks")
    LA = torch.empty((n, n), dtype=A.dtype, device=dev)
    LB = torch.empty((heads, b, b), dtype=A.dtype, device=dev)
    dA = torch.empty(n, dtype=A.dtype, device=dev)
    dB = torch.empty(heads * b, dtype=A.dtype, device=dev)
    L = lib()
    ws = _workspace(L.bakron_factor_blockdiag_workspace_bytes(code, heads, heads * b, n), dev, workspace)
    bad = (_i64 * 3)(-1, -1, -1)
    with torch.cuda.device(dev):
        rc = L.bakron_factor_blockdiag(code, heads, heads * b, n, _p(A), _ld(A, "A"), pb, ldb, sb,
                                       _p(LA), max(n, 1), _p(LB), max(b, 1), b * b, _p(dA), _p(dB),
                                       _p(ws), ws.numel() * ws.element_size(), bad, _stream(dev))
    if rc != OK:
        err = BakronError(rc, "bakron_factor_blockdiag")
        err.bad_pivot = (int(bad[0]), int(bad[1]), int(bad[2]))
        raise err
    return LA, LB, dA, dB


def solve_blockdiag(W: torch.Tensor, LA: torch.Tensor, LBblocks: torch.Tensor,
                    alphabet: AlphabetLike = (0, 0, 1), scales: Optional[torch.Tensor] = None,
                    scale_mode: Optional[int] = None, return_wt: bool = False,
                    workspace: Optional[torch.Tensor] = None, check: bool = False):
    """The BaKron solve with a block-diagonal L^B given by its blocks
    (heads, b, b), m = heads * b: all heads in the same launches. ``check``:
    as in ``solve``."""
    dev = _check_device(W, LA, LBblocks, scales, workspace)
    code = _dt(W)
    m, n = W.shape
    if LBblocks.dim() != 3 or LBblocks.size(0) * LBblocks.size(1) != m:
        raise ValueError("LBblocks must be (heads, b, b) with heads * b = m")
    heads, b = LBblocks.size(0), LBblocks.size(1)
    if LA.shape != (n, n) or LA.dtype != W.dtype or LBblocks.dtype != W.dtype:
        raise ValueError("LA must be n x n, all of W's dtype")
    plb, ldlb, slb = _blocks(LBblocks, heads, b, "LBblocks")
    lo, hi, unb = (int(alphabet[0]), int(alphabet[1]), int(bool(alphabet[2])))
    mode = _scale_mode(scales, m, n, scale_mode)
    if scales is not None and (scales.dtype != W.dtype or not scales.is_contiguous()):
        raise ValueError("scales must be contiguous with W's dtype")
    V = torch.empty((m, n), dtype=torch.int32, device=dev)
    Wt = torch.empty((m, n), dtype=W.dtype, device=dev) if return_wt else None
    L = lib()
    ws = _workspace(L.bakron_solve_blockdiag_workspace_bytes(code, heads, m, n), dev, workspace)
    with torch.cuda.device(dev):
        rc = L.bakron_solve_blockdiag(code, heads, m, n, _p(W), _ld(W, "W"), _p(LA), _ld(LA, "LA"),
                                      plb, ldlb, slb, lo, hi, unb, mode, _p(scales), _p(V),
                                      _ld(V, "V"), _p(Wt), _ld(Wt, "Wt") if Wt is not None else 0,
                                      _p(ws), ws.numel() * ws.element_size(), _stream(dev))
    if rc == OK and check:
        rc = L.bakron_solve_status(code, heads, b, n, _p(ws), ws.numel() * ws.element_size(),
                                   _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_solve_blockdiag")
    return (V, Wt) if return_wt else V


def loss_blockdiag(W: torch.Tensor, V: torch.Tensor, A: torch.Tensor, Bblocks: torch.Tensor,
                   scales: Optional[torch.Tensor] = None, scale_mode: Optional[int] = None,
                   workspace: Optional[torch.Tensor] = None, sync: bool = True):
    """tr(B (W - s V) A (W - s V)^T) for B = blockdiag(Bblocks[h]), in float64."""
    dev = _check_device(W, V, A, Bblocks, scales, workspace)
    code = _dt(W)
    m, n = W.shape
    if Bblocks.dim() != 3 or Bblocks.size(0) * Bblocks.size(1) != m:
        raise ValueError("Bblocks must be (heads, b, b) with heads * b = m")
    heads, b = Bblocks.size(0), Bblocks.size(1)
    _check_operand(V, (m, n), torch.int32, "V")
    _check_operand(A, (n, n), W.dtype, "A")
    if Bblocks.dtype != W.dtype:
        raise TypeError("Bblocks must have W's dtype")
    pb, ldb, sb = _blocks(Bblocks, heads, b, "Bblocks")
    mode = _scale_mode(scales, m, n, scale_mode)
    if scales is not None and (scales.dtype != W.dtype or not scales.is_contiguous()):
        raise ValueError("scales must be contiguous with W's dtype")
    out = torch.zeros(1, dtype=torch.float64, device=dev)
    L = lib()
    ws = _workspace(L.bakron_loss_blockdiag_workspace_bytes(code, heads, m, n), dev, workspace)
    with torch.cuda.device(dev):
        rc = L.bakron_loss_blockdiag(code, heads, m, n, _p(W), _ld(W, "W"), _p(V), _ld(V, "V"), mode,
                                     _p(scales), _p(A), _ld(A, "A"), pb, ldb, sb, _p(out), _p(ws),
                                     ws.numel() * ws.element_size(), _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_loss_blockdiag")
    return float(out.item()) if sync else out


# Largest workspace bakron_solve_noalloc takes from its in-library scratch
# (BAKRON_NOALLOC_SCRATCH_BYTES in include/bakron.h).
NOALLOC_SCRATCH_BYTES = 96 << 20


def solve_noalloc(W: torch.Tensor, LA: torch.Tensor, LB: torch.Tensor, alphabet: AlphabetLike,
                  scales: Optional[torch.Tensor], V: torch.Tensor, Wt: Optional[torch.Tensor] = None,
                  scale_mode: Optional[int] = None, check: bool = False) -> torch.Tensor:
    """bakron_solve_noalloc: the solve of ``solve`` with the library's own
    per-GPU scratch instead of a workspace. The caller passes the outputs
    (V int32 m x n, optional Wt of W's dtype); nothing is allocated. Calls
    that overlap on one GPU race on the scratch. ``check``: as in ``solve``."""
    dev = _check_device(W, LA, LB, scales, V, Wt)
    code = _dt(W)
    m, n = W.shape
    if LA.shape != (n, n) or LB.shape != (m, m) or LA.dtype != W.dtype or LB.dtype != W.dtype:
        raise ValueError("LA must be n x n and LB m x m, same dtype as W")
    lo, hi, unb = (int(alphabet[0]), int(alphabet[1]), int(bool(alphabet[2])))
    mode = _scale_mode(scales, m, n, scale_mode)
    if scales is not None and (scales.dtype != W.dtype or not scales.is_contiguous()):
        raise ValueError("scales must be contiguous with W's dtype")
    _check_out(V, (m, n), torch.int32, "V")
    if Wt is not None:
        _check_out(Wt, (m, n), W.dtype, "Wt")
    with torch.cuda.device(dev):
        rc = lib().bakron_solve_noalloc(code, m, n, _p(W), _ld(W, "W"), _p(LA), _ld(LA, "LA"),
                                        _p(LB), _ld(LB, "LB"), lo, hi, unb, mode, _p(scales),
                                        _p(V), _ld(V, "V"), _p(Wt),
                                        _ld(Wt, "Wt") if Wt is not None else 0, _stream(dev))
    if rc == OK and check:
        with torch.cuda.device(dev):
            rc = lib().bakron_solve_status(code, 1, m, n, None, 0, _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_solve_noalloc")
    return V


def _batch_operand(t: torch.Tensor, rows: int, cols: int, batch: int, name: str):
    """(pointer, ld, stride) of a batched operand: a (batch, rows, cols)
    tensor, or a single (rows, cols) matrix shared by every problem."""
    if t.dim() == 2:
        if t.shape != (rows, cols):
            raise ValueError(f"{name} must be {rows} x {cols}")
        return _p(t), _ld(t, name), 0
    if t.dim() != 3 or t.shape != (batch, rows, cols):
        raise ValueError(f"{name} must be ({batch}, {rows}, {cols}) or ({rows}, {cols})")
    if cols > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    ld = max(int(t.stride(1)), cols, 1)
    return _p(t), ld, int(t.stride(0)) if batch > 1 else 0


def solve_batched(W: torch.Tensor, LA: torch.Tensor, LB: torch.Tensor,
                  alphabet: AlphabetLike = (0, 0, 1), scales: Optional[torch.Tensor] = None,
                  scale_mode: Optional[int] = None, return_wt: bool = False,
                  workspace: Optional[torch.Tensor] = None, check: bool = False):
    """bakron_solve on a batch of problems of one shape in the same launches.
    W is (batch, m, n); LA is (batch, n, n) or one (n, n) factor shared by
    all problems, LB likewise (batch, m, m) or (m, m); scales (batch, m) /
    (batch, n) or one shared vector. Returns int32 codes (batch, m, n) and,
    with ``return_wt``, the values at rounding. Each problem's result equals
    ``solve`` on the same inputs bit for bit. ``check``: as in ``solve``."""
    dev = _check_device(W, LA, LB, scales, workspace)
    code = _dt(W)
    if W.dim() != 3:
        raise ValueError("W must be (batch, m, n)")
    batch, m, n = W.shape
    if LA.dtype != W.dtype or LB.dtype != W.dtype:
        raise ValueError("LA and LB must have W's dtype")
    pw, ldw, sw = _batch_operand(W, m, n, batch, "W")
    pla, ldla, sla = _batch_operand(LA, n, n, batch, "LA")
    plb, ldlb, slb = _batch_operand(LB, m, m, batch, "LB")
    lo, hi, unb = (int(alphabet[0]), int(alphabet[1]), int(bool(alphabet[2])))
    ss = 0
    if scales is None:
        if scale_mode not in (None, SCALE_NONE):
            raise ValueError("scales required for this scale_mode")
        mode = SCALE_NONE
    else:
        if scales.dtype != W.dtype or not scales.is_contiguous():
            raise ValueError("scales must be contiguous with W's dtype")
        vec = scales if scales.dim() == 1 else scales[0]
        if scales.dim() not in (1, 2) or (scales.dim() == 2 and scales.size(0) != batch):
            raise ValueError("scales must be (batch, length) or (length,)")
        mode = _scale_mode(vec, m, n, scale_mode)
        ss = int(scales.stride(0)) if scales.dim() == 2 and batch > 1 else 0
    V = torch.empty((batch, m, n), dtype=torch.int32, device=dev)
    Wt = torch.empty((batch, m, n), dtype=W.dtype, device=dev) if return_wt else None
    L = lib()
    ws = _workspace(L.bakron_solve_batched_workspace_bytes(code, batch, m, n), dev, workspace)
    with torch.cuda.device(dev):
        rc = L.bakron_solve_batched(code, batch, m, n, pw, ldw, sw, pla, ldla, sla, plb, ldlb, slb,
                                    lo, hi, unb, mode, _p(scales), ss, _p(V), max(n, 1), m * n,
                                    _p(Wt), max(n, 1) if return_wt else 0,
                                    m * n if return_wt else 0, _p(ws),
                                    ws.numel() * ws.element_size(), _stream(dev))
    if rc == OK and check:
        rc = L.bakron_solve_status(code, batch, m, n, _p(ws), ws.numel() * ws.element_size(),
                                   _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_solve_batched")
    return (V, Wt) if return_wt else V


def loss(W: torch.Tensor, V: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
         scales: Optional[torch.Tensor] = None, scale_mode: Optional[int] = None,
         workspace: Optional[torch.Tensor] = None, sync: bool = True):
    """tr(B (W - s V) A (W - s V)^T) in float64 (Proposition 3.1). Returns a
    Python float (``sync``) or a 1-element float64 device tensor."""
    dev = _check_device(W, V, A, B, scales, workspace)
    code = _dt(W)
    m, n = W.shape
    mode = _scale_mode(scales, m, n, scale_mode)
    _check_operand(V, (m, n), torch.int32, "V")
    _check_operand(A, (n, n), W.dtype, "A")
    _check_operand(B, (m, m), W.dtype, "B")
    if scales is not None and (scales.dtype != W.dtype or not scales.is_contiguous()):
        raise ValueError("scales must be contiguous with W's dtype")
    out = torch.zeros(1, dtype=torch.float64, device=dev)
    L = lib()
    ws = _workspace(L.bakron_loss_workspace_bytes(code, m, n), dev, workspace)
    with torch.cuda.device(dev):
        rc = L.bakron_loss(code, m, n, _p(W), _ld(W, "W"), _p(V), _ld(V, "V"), mode, _p(scales),
                           _p(A), _ld(A, "A"), _p(B), _ld(B, "B"), _p(out), _p(ws),
                           ws.numel() * ws.element_size(), _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_loss")
    return float(out.item()) if sync else out


def loss_batched(W: torch.Tensor, V: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                 scales: Optional[torch.Tensor] = None, scale_mode: Optional[int] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bakron_loss for a batch in the same launches: W, V (batch, m, n); A
    (batch, n, n) or one (n, n); B (batch, m, m) or one (m, m); scales
    (batch, length) or one vector. Returns a float64 device tensor of
    ``batch`` losses (asynchronous)."""
    dev = _check_device(W, V, A, B, scales, workspace)
    code = _dt(W)
    if W.dim() != 3 or V.dim() != 3 or V.shape != W.shape or V.dtype != torch.int32:
        raise ValueError("W and V must be (batch, m, n), V int32")
    batch, m, n = W.shape
    if A.dtype != W.dtype or B.dtype != W.dtype:
        raise TypeError("A and B must have W's dtype")
    pw, ldw, sw = _batch_operand(W, m, n, batch, "W")
    pv, ldv, sv = _batch_operand(V, m, n, batch, "V")
    pa, lda, sa = _batch_operand(A, n, n, batch, "A")
    pb, ldb, sb = _batch_operand(B, m, m, batch, "B")
    ss = 0
    if scales is None:
        if scale_mode not in (None, SCALE_NONE):
            raise ValueError("scales required for this scale_mode")
        mode = SCALE_NONE
    else:
        if scales.dtype != W.dtype or not scales.is_contiguous():
            raise ValueError("scales must be contiguous with W's dtype")
        if scales.dim() not in (1, 2) or (scales.dim() == 2 and scales.size(0) != batch):
            raise ValueError("scales must be (batch, length) or (length,)")
        vec = scales if scales.dim() == 1 else scales[0]
        mode = _scale_mode(vec, m, n, scale_mode)
        ss = int(scales.stride(0)) if scales.dim() == 2 and batch > 1 else 0
    out = torch.zeros(batch, dtype=torch.float64, device=dev)
    L = lib()
    ws = _workspace(L.bakron_loss_batched_workspace_bytes(code, batch, m, n), dev, workspace)
    with torch.cuda.device(dev):
        rc = L.bakron_loss_batched(code, batch, m, n, pw, ldw, sw, pv, ldv, sv, mode, _p(scales), ss,
                                   pa, lda, sa, pb, ldb, sb, _p(out), _p(ws),
                                   ws.numel() * ws.element_size(), _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_loss_batched")
    return out


def row_scales(W: torch.Tensor, hi: int) -> torch.Tensor:
    """s_i = max_j |W_ij| / hi (1 for an all-zero row), in W's dtype."""
    dev = _check_device(W)
    code = _dt(W)
    m, n = W.shape
    s = torch.empty(m, dtype=W.dtype, device=dev)
    with torch.cuda.device(dev):
        rc = lib().bakron_row_scales(code, m, n, _p(W), _ld(W, "W"), int(hi), _p(s), _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_row_scales")
    return s


def row_scales_mse(W: torch.Tensor, alphabet: AlphabetLike, grid: int = 100,
                   max_shrink: float = 0.5) -> torch.Tensor:
    """Per-row absmax / hi scales shrunk by up to 1 / (1 - max_shrink) by a
    search over grid + 1 candidates for the smallest round-to-nearest squared
    error of the row (bakron_row_scales_mse), in W's dtype."""
    dev = _check_device(W)
    code = _dt(W)
    m, n = W.shape
    lo, hi = int(alphabet[0]), int(alphabet[1])
    s = torch.empty(m, dtype=W.dtype, device=dev)
    with torch.cuda.device(dev):
        rc = lib().bakron_row_scales_mse(code, m, n, _p(W), _ld(W, "W"), lo, hi, int(grid),
                                         float(max_shrink), _p(s), _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_row_scales_mse")
    return s


def gram(X: torch.Tensor, weights: Optional[torch.Tensor] = None, damp_rel: float = 0.0,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """(1/N) sum_k w_k x_k x_k^T over the rows of X (N x d), plus
    damp_rel * mean(diag) * I (bakron_gram): the K-FAC factor with no
    weights, the one-step Shampoo factor with the other side's squared norms."""
    dev = _check_device(X, weights, out)
    code = _dt(X)
    N, d = X.shape
    if weights is not None and (weights.dtype != X.dtype or weights.numel() != N
                                or not weights.is_contiguous()):
        raise ValueError("weights must be a contiguous length-N vector of X's dtype")
    if out is not None:
        _check_out(out, (d, d), X.dtype, "out")
    G = out if out is not None else torch.empty((d, d), dtype=X.dtype, device=dev)
    with torch.cuda.device(dev):
        rc = lib().bakron_gram(code, N, d, _p(X), _ld(X, "X"), _p(weights), float(damp_rel),
                               _p(G), _ld(G, "G"), _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_gram")
    return G


def sample_sqnorms(X: torch.Tensor) -> torch.Tensor:
    """|x_k|^2 of every row of X (bakron_sample_sqnorms)."""
    dev = _check_device(X)
    code = _dt(X)
    N, d = X.shape
    out = torch.empty(N, dtype=X.dtype, device=dev)
    with torch.cuda.device(dev):
        rc = lib().bakron_sample_sqnorms(code, N, d, _p(X), _ld(X, "X"), _p(out), _stream(dev))
    if rc != OK:
        raise BakronError(rc, "bakron_sample_sqnorms")
    return out


def kfac_factors(Xa: torch.Tensor, Xb: torch.Tensor, damp_rel: float = 0.0):
    """K-FAC-style Kronecker factors A = E[a a^T], B = E[b b^T] (§4.2) from
    the sample rows of Xa (N x n) and Xb (N x m)."""
    return gram(Xa, None, damp_rel), gram(Xb, None, damp_rel)


def shampoo_factors(Xa: torch.Tensor, Xb: torch.Tensor, damp_rel: float = 0.0):
    """One-step Shampoo-style factors A = E[|b|^2 a a^T], B = E[|a|^2 b b^T]
    (§4.2, Appendix A.2)."""
    return gram(Xa, sample_sqnorms(Xb), damp_rel), gram(Xb, sample_sqnorms(Xa), damp_rel)


def debug_set_wait_polls(polls: int) -> int:
    """Test hook: the poll bound of the leaf blocks' waits for solves enqueued
    from now on (negative: the default); returns the previous bound."""
    return int(lib().bakron_debug_set_wait_polls(int(polls)))


def solve_schedule(dtype: int, m: int, n: int):
    """The solve's launch schedule: list of (kind, a, b, c); kind 0 = leaf
    block of tile anti-diagonals [a, b), kinds 2/3 = the two band products of
    the internal node [a, b) -> [b, c). Host only."""
    L = lib()
    cnt = int(L.bakron_solve_schedule(int(dtype), int(m), int(n), None, 0))
    if cnt < 0:
        raise BakronError(cnt, "bakron_solve_schedule")
    buf = (ctypes.c_int32 * (4 * max(cnt, 1)))()
    L.bakron_solve_schedule(int(dtype), int(m), int(n), ctypes.cast(buf, ctypes.c_void_p), cnt)
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(cnt)]
