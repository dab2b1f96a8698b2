"""Python binding of libwq.so: fused low-bit dequantize-and-multiply on MI355X.

Argument marshalling only.  Every step of every product runs in the HIP
kernels of libwq.so; torch supplies device memory and the current stream.
There is no fallback: without the built library every call raises.

Entry points (same names as the C ABI in ``include/wq.h``).  The weight-only
products read a packed copy of the weight made once by ``prepack_*``:

* ``prepack_q3(qweight, K)`` / ``matvec_q3(x, packed, scales, zeros)``       -> y
* ``prepack_q8(qweight)`` / ``gemm_q8_group(X, packed, scales, group_size)``  -> Y
* ``q4_act_order_perm(g_idx, K, G)`` -> (perm, invperm) host int32 arrays
* ``prepack_q4(qweight, perm, G)`` / ``gemm_q4_group(X, packed, scales, invperm, G)`` -> Y
  (``prepare_q4(qweight, g_idx, G)`` does the act-order preparation in one go)
* ``prepare_q2(qweight, g_idx, G)`` / ``gemm_q2_group_zp(X, packed, scales, zeros, G)`` -> Y
  (asymmetric 2-bit, 16 codes per int32 along K)
* ``gemm_w8a8(X, Wq, Sw, want_acc=False)``  -> (Y bf16, Xq, Sx, acc | None)
* ``unpack_q3`` / ``unpack_q8`` / ``unpack_q4``: codes held by a packed weight
* ``calib_empty`` / ``calib_stream_read``: timing references (no product)
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "wq.h")

WQ_OK, WQ_ERR_NULL, WQ_ERR_SHAPE, WQ_ERR_ALIGN, WQ_ERR_DTYPE, WQ_ERR_WORKSPACE, WQ_ERR_HIP = 0, 1, 2, 3, 4, 5, 6
WQ_F32, WQ_F16 = 0, 1
WQ_OP_Q3, WQ_OP_Q4G, WQ_OP_Q8G, WQ_OP_Q2G, WQ_OP_W8A8 = 0, 1, 2, 3, 4

_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGNATURES = {
    "wq_packed_bytes": (_sz, [_i, _i, _i, _i]),
    "wq_prepack_q3": (_i, [_vp, _vp, _i, _i, _vp]),
    "wq_matvec_q3": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "wq_prepack_q8": (_i, [_vp, _vp, _i, _i, _vp]),
    "wq_gemm_q8_group": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "wq_dequant_q8_group": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "wq_q4_act_order_perm": (_i, [_vp, _i, _i, _vp, _vp]),
    "wq_prepack_q4": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp]),
    "wq_gemm_q4_group": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "wq_gemm_q4_group_zp": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "wq_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "wq_gemm_w8a8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _vp]),
    "wq_gemm_w8a8_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "wq_gemm_w8a8_smooth": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i, _i, _i, _vp]),
    "wq_gemm_int8_mixed": (_i, [_vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _sz, _i, _i, _i, _vp]),
    "wq_prepack_q2": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp]),
    "wq_gemm_q2_group_zp": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "wq_unpack_q2": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp]),
    "wq_unpack_q3": (_i, [_vp, _vp, _i, _i, _vp]),
    "wq_unpack_q8": (_i, [_vp, _vp, _i, _i, _vp]),
    "wq_unpack_q4": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp]),
    "wq_calib_empty": (_i, [_i, _i, _vp, _vp]),
    "wq_calib_stream_read": (_i, [_vp, ctypes.c_longlong, _vp, _vp]),
    "wq_status_str": (ctypes.c_char_p, [_i]),
    "wq_last_hip_error": (_i, []),
}

_lib = None


class WQError(RuntimeError):
    """A libwq call returned a non-OK status."""

    def __init__(self, fn: str, status: int, text: str, hip: int = 0):
        msg = f"{fn}: {text} (status {status})"
        if status == WQ_ERR_HIP:
            msg += f", hipError_t {hip}"
        super().__init__(msg)
        self.status = status


def header_functions() -> list[str]:
    """Names of the functions ``include/wq.h`` declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(wq_\w+)\s*\(", text, re.M)))


def lib() -> ctypes.CDLL:
    """The loaded library (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, st: int) -> None:
    if st != WQ_OK:
        L = lib()
        raise WQError(fn, st, L.wq_status_str(st).decode(), L.wq_last_hip_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def packed_bytes(op: int, K: int, N: int, G: int = 0) -> int:
    n = int(lib().wq_packed_bytes(op, K, N, G))
    if n == 0:
        _check("wq_packed_bytes", WQ_ERR_SHAPE)
    return n


def _packed(op, K, N, G, device):
    return torch.empty(packed_bytes(op, K, N, G), dtype=torch.uint8, device=device)


def _need_packed(t, op, K, N, G, device):
    _need(t, "packed", torch.uint8, (packed_bytes(op, K, N, G),), device)


# ----------------------------------------------------------------- 3-bit --

def prepack_q3(qweight, K: int):
    """Re-lay out a 3-bit weight [3K/32, N] int32 for matvec_q3."""
    N = qweight.shape[1]
    dev = qweight.device
    _need(qweight, "qweight", torch.int32, (3 * K // 32, N), dev)
    out = _packed(WQ_OP_Q3, K, N, 0, dev)
    _check("wq_prepack_q3", lib().wq_prepack_q3(_ptr(qweight), _ptr(out), K, N, _stream(dev)))
    return out


def matvec_q3(x, packed, scales, zeros, y=None):
    """y = x . (scale * q - zero) from a packed 3-bit weight; fp32 or fp16."""
    K, N = x.shape[0], scales.shape[0]
    dt = x.dtype
    if dt not in (torch.float32, torch.float16):
        raise TypeError("x must be float32 or float16")
    dev = x.device
    _need(x, "x", dt, (K,), dev)
    _need_packed(packed, WQ_OP_Q3, K, N, 0, dev)
    _need(scales, "scales", dt, (N,), dev)
    _need(zeros, "zeros", dt, (N,), dev)
    if y is None:
        y = torch.empty(N, dtype=dt, device=dev)
    _need(y, "y", dt, (N,), dev)
    st = lib().wq_matvec_q3(_ptr(x), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(y), K, N,
                            WQ_F16 if dt == torch.float16 else WQ_F32, _stream(dev))
    _check("wq_matvec_q3", st)
    return y


def unpack_q3(packed, K: int, N: int):
    dev = packed.device
    _need_packed(packed, WQ_OP_Q3, K, N, 0, dev)
    codes = torch.empty((K, N), dtype=torch.int8, device=dev)
    _check("wq_unpack_q3", lib().wq_unpack_q3(_ptr(packed), _ptr(codes), K, N, _stream(dev)))
    return codes


# ------------------------------------------------------------------ int8 --

def prepack_q8(qweight):
    """Re-lay out a group-wise int8 weight [K, N] for gemm_q8_group."""
    K, N = qweight.shape
    dev = qweight.device
    _need(qweight, "qweight", torch.int8, (K, N), dev)
    out = _packed(WQ_OP_Q8G, K, N, 0, dev)
    _check("wq_prepack_q8", lib().wq_prepack_q8(_ptr(qweight), _ptr(out), K, N, _stream(dev)))
    return out


def gemm_q8_group(X, packed, scales, group_size=128, Y=None, ws=None):
    """Y = X . (scale[k // G] * q) from a packed int8 weight; X fp16 [M, K] or [K].

    ``ws``: device workspace of ``workspace_bytes(WQ_OP_Q8G, M, K, N)`` bytes
    (K split over workgroups above 32 rows), allocated here if None and needed.
    """
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    M, K = X2.shape
    N = scales.shape[1]
    dev = X.device
    _need(X2, "X", torch.float16, (M, K), dev)
    _need_packed(packed, WQ_OP_Q8G, K, N, 0, dev)
    _need(scales, "scales", torch.float32, (K // group_size, N), dev)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(Y, "Y", torch.float16, (M, N), dev)
    ws, nws = _workspace_op(WQ_OP_Q8G, ws, M, K, N, dev)
    st = lib().wq_gemm_q8_group(_ptr(X2), _ptr(packed), _ptr(scales), _ptr(Y), M, K, N,
                                group_size, _ptr(ws) if ws is not None else None, nws, _stream(dev))
    _check("wq_gemm_q8_group", st)
    return Y.reshape(N) if squeeze else Y


def dequant_q8_group(qweight, scales, group_size=128, dtype=torch.float32, W=None):
    """The separated form's dequantisation: ``W = scale[k // G] * q`` as a dense
    fp32 (or fp16) [K, N] weight, from the stored int8 codes [K, N]."""
    K, N = qweight.shape
    dev = qweight.device
    _need(qweight, "qweight", torch.int8, (K, N), dev)
    _need(scales, "scales", torch.float32, (K // group_size, N), dev)
    if dtype not in (torch.float32, torch.float16):
        raise ValueError("dtype must be torch.float32 or torch.float16")
    if W is None:
        W = torch.empty((K, N), dtype=dtype, device=dev)
    _need(W, "W", dtype, (K, N), dev)
    st = lib().wq_dequant_q8_group(_ptr(qweight), _ptr(scales), _ptr(W), K, N, group_size,
                                   WQ_F32 if dtype == torch.float32 else WQ_F16, _stream(dev))
    _check("wq_dequant_q8_group", st)
    return W


def unpack_q8(packed, K: int, N: int):
    dev = packed.device
    _need_packed(packed, WQ_OP_Q8G, K, N, 0, dev)
    codes = torch.empty((K, N), dtype=torch.int8, device=dev)
    _check("wq_unpack_q8", lib().wq_unpack_q8(_ptr(packed), _ptr(codes), K, N, _stream(dev)))
    return codes


# ----------------------------------------------------------------- 4-bit --

def q4_act_order_perm(g_idx, K: int, group_size: int = 128):
    """Host: (perm, invperm), rows listed group by group; ``g_idx=None`` is the identity."""
    perm = np.empty(K, dtype=np.int32)
    inv = np.empty(K, dtype=np.int32)
    pp, ip = perm.ctypes.data_as(ctypes.c_void_p), inv.ctypes.data_as(ctypes.c_void_p)
    if g_idx is None:
        st = lib().wq_q4_act_order_perm(None, K, group_size, pp, ip)
    else:
        g = np.ascontiguousarray(np.asarray(g_idx.cpu() if isinstance(g_idx, torch.Tensor) else g_idx,
                                            dtype=np.int32))
        if g.shape != (K,):
            raise ValueError(f"g_idx must have shape ({K},)")
        st = lib().wq_q4_act_order_perm(g.ctypes.data_as(ctypes.c_void_p), K, group_size, pp, ip)
    _check("wq_q4_act_order_perm", st)
    return perm, inv


def _check_perm(perm, K):
    """``perm`` must list every row 0..K-1 exactly once (checked on the host)."""
    p = perm.cpu().numpy()
    if not np.array_equal(np.sort(p), np.arange(K, dtype=p.dtype)):
        raise ValueError("perm must be a permutation of 0..K-1")


def prepack_q4(qweight, perm=None, group_size=128):
    """Device: re-lay out a 4-bit weight [K/8, N], rows in ``perm`` order (or as stored)."""
    R, N = qweight.shape
    K = 8 * R
    dev = qweight.device
    _need(qweight, "qweight", torch.int32, (R, N), dev)
    if perm is not None:
        _need(perm, "perm", torch.int32, (K,), dev)
        _check_perm(perm, K)
    out = _packed(WQ_OP_Q4G, K, N, group_size, dev)
    st = lib().wq_prepack_q4(_ptr(qweight), _ptr(perm), _ptr(out), K, N, group_size, _stream(dev))
    _check("wq_prepack_q4", st)
    return out


def prepare_q4(qweight, g_idx, group_size=128):
    """Act-order preparation in one go: ``(packed, perm_dev)``.

    The packed weight carries the row order (its inverse, as a row table), so
    the product needs nothing else.  With ``g_idx=None`` the stored order is
    kept and ``perm_dev`` is None.
    """
    if g_idx is None:
        return prepack_q4(qweight, None, group_size), None
    K = 8 * qweight.shape[0]
    perm, _ = q4_act_order_perm(g_idx, K, group_size)
    perm_d = torch.from_numpy(perm).to(qweight.device)
    return prepack_q4(qweight, perm_d, group_size), perm_d


def _workspace_q4(ws, M, K, N, dev):
    return _workspace_op(WQ_OP_Q4G, ws, M, K, N, dev)


def _workspace_op(op, ws, M, K, N, dev):
    need = workspace_bytes(op, M, K, N)
    if ws is None:
        if need == 0:
            return None, 0
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if not (ws.is_cuda and ws.is_contiguous() and ws.device == dev):
        raise ValueError("ws must be a contiguous tensor on the device of X")
    return ws, ws.numel() * ws.element_size()


def gemm_q4_group(X, packed, scales, group_size=128, Y=None, ws=None):
    """Y[m, n] = sum_k X[m, k] * scale[g_idx[k], n] * q[k, n] from a packed 4-bit weight.

    ``ws``: device workspace of ``workspace_bytes(WQ_OP_Q4G, M, K, N)`` bytes
    (needed above 4 rows of X; allocated here if None).
    """
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    M, K = X2.shape
    N = scales.shape[1]
    dev = X.device
    _need(X2, "X", torch.float16, (M, K), dev)
    _need_packed(packed, WQ_OP_Q4G, K, N, group_size, dev)
    _need(scales, "scales", torch.float16, (K // group_size, N), dev)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(Y, "Y", torch.float16, (M, N), dev)
    ws, ws_bytes = _workspace_q4(ws, M, K, N, dev)
    st = lib().wq_gemm_q4_group(_ptr(X2), _ptr(packed), _ptr(scales), _ptr(Y), M, K, N, group_size,
                                _ptr(ws), ws_bytes, _stream(dev))
    _check("wq_gemm_q4_group", st)
    return Y.reshape(N) if squeeze else Y


def gemm_q4_group_zp(X, packed, scales, zeros, group_size=128, Y=None, ws=None):
    """Y[m, n] = sum_k X[m, k] * (u[k, n] - zero[g, n]) * scale[g, n] (asymmetric 4-bit)."""
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    M, K = X2.shape
    N = scales.shape[1]
    dev = X.device
    _need(X2, "X", torch.float16, (M, K), dev)
    _need_packed(packed, WQ_OP_Q4G, K, N, group_size, dev)
    _need(scales, "scales", torch.float16, (K // group_size, N), dev)
    _need(zeros, "zeros", torch.float16, (K // group_size, N), dev)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(Y, "Y", torch.float16, (M, N), dev)
    ws, ws_bytes = _workspace_q4(ws, M, K, N, dev)
    st = lib().wq_gemm_q4_group_zp(_ptr(X2), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(Y), M, K,
                                   N, group_size, _ptr(ws), ws_bytes, _stream(dev))
    _check("wq_gemm_q4_group_zp", st)
    return Y.reshape(N) if squeeze else Y


def unpack_q4(packed, K: int, N: int, group_size: int = 128, perm=None):
    dev = packed.device
    _need_packed(packed, WQ_OP_Q4G, K, N, group_size, dev)
    if perm is not None:
        _need(perm, "perm", torch.int32, (K,), dev)
    codes = torch.empty((K, N), dtype=torch.int8, device=dev)
    _check("wq_unpack_q4", lib().wq_unpack_q4(_ptr(packed), _ptr(perm), _ptr(codes), K, N,
                                              group_size, _stream(dev)))
    return codes


# ----------------------------------------------------------------- 2-bit --

def prepack_q2(qweight, perm=None, group_size=128):
    """Device: re-lay out a 2-bit weight [K/16, N], rows in ``perm`` order (or as stored)."""
    R, N = qweight.shape
    K = 16 * R
    dev = qweight.device
    _need(qweight, "qweight", torch.int32, (R, N), dev)
    if perm is not None:
        _need(perm, "perm", torch.int32, (K,), dev)
        _check_perm(perm, K)
    out = _packed(WQ_OP_Q2G, K, N, group_size, dev)
    st = lib().wq_prepack_q2(_ptr(qweight), _ptr(perm), _ptr(out), K, N, group_size, _stream(dev))
    _check("wq_prepack_q2", st)
    return out


def prepare_q2(qweight, g_idx, group_size=128):
    """Act-order preparation and re-layout of a 2-bit weight: ``(packed, perm_dev)``."""
    if g_idx is None:
        return prepack_q2(qweight, None, group_size), None
    K = 16 * qweight.shape[0]
    perm, _ = q4_act_order_perm(g_idx, K, group_size)
    perm_d = torch.from_numpy(perm).to(qweight.device)
    return prepack_q2(qweight, perm_d, group_size), perm_d


def gemm_q2_group_zp(X, packed, scales, zeros, group_size=128, Y=None):
    """Y[m, n] = sum_k X[m, k] * (u[k, n] - zero[g, n]) * scale[g, n] (asymmetric 2-bit)."""
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    M, K = X2.shape
    N = scales.shape[1]
    dev = X.device
    _need(X2, "X", torch.float16, (M, K), dev)
    _need_packed(packed, WQ_OP_Q2G, K, N, group_size, dev)
    _need(scales, "scales", torch.float16, (K // group_size, N), dev)
    _need(zeros, "zeros", torch.float16, (K // group_size, N), dev)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(Y, "Y", torch.float16, (M, N), dev)
    st = lib().wq_gemm_q2_group_zp(_ptr(X2), _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(Y), M, K,
                                   N, group_size, _stream(dev))
    _check("wq_gemm_q2_group_zp", st)
    return Y.reshape(N) if squeeze else Y


def unpack_q2(packed, K: int, N: int, group_size: int = 128, perm=None):
    """The values u (0..3) a packed 2-bit weight holds, in the original row order."""
    dev = packed.device
    _need_packed(packed, WQ_OP_Q2G, K, N, group_size, dev)
    if perm is not None:
        _need(perm, "perm", torch.int32, (K,), dev)
    codes = torch.empty((K, N), dtype=torch.int8, device=dev)
    _check("wq_unpack_q2", lib().wq_unpack_q2(_ptr(packed), _ptr(perm), _ptr(codes), K, N,
                                              group_size, _stream(dev)))
    return codes


# ------------------------------------------------------------------ W8A8 --

def workspace_bytes(op: int, M: int, K: int, N: int) -> int:
    """Device workspace bytes a call of ``op`` needs at this shape (0 if none)."""
    return int(lib().wq_workspace_bytes(op, M, K, N))


def _workspace(ws, M, K, N, dev):
    need = workspace_bytes(WQ_OP_W8A8, M, K, N)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if not (ws.is_cuda and ws.is_contiguous() and ws.device == dev):
        raise ValueError("ws must be a contiguous tensor on the device of X")
    return ws, ws.numel() * ws.element_size()


def gemm_w8a8(X, Wq, Sw, want_acc=False, Y=None, Xq=None, Sx=None, acc=None, smooth=None, ws=None):
    """Dynamic W8A8: returns ``(Y bf16 [M,N], Xq int8 [M,K], Sx fp32 [M], acc int32 | None)``.

    With ``smooth`` (fp32 [K]) the SmoothQuant entry point runs instead: X is
    divided by it per input channel before quantisation, and Wq, Sw must
    quantise ``diag(smooth) . W``.  ``ws``: a device workspace of at least
    ``workspace_bytes(WQ_OP_W8A8, M, K, N)`` bytes, allocated here if None.
    """
    M, K = X.shape
    N = Wq.shape[0]
    dev = X.device
    _need(X, "X", torch.float32, (M, K), dev)
    _need(Wq, "Wq", torch.int8, (N, K), dev)
    _need(Sw, "Sw", torch.float32, (N,), dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if Y is None else Y
    Xq = torch.empty((M, K), dtype=torch.int8, device=dev) if Xq is None else Xq
    Sx = torch.empty(M, dtype=torch.float32, device=dev) if Sx is None else Sx
    if want_acc and acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    _need(Y, "Y", torch.bfloat16, (M, N), dev)
    _need(Xq, "Xq", torch.int8, (M, K), dev)
    _need(Sx, "Sx", torch.float32, (M,), dev)
    if acc is not None:
        _need(acc, "acc", torch.int32, (M, N), dev)
    ws, ws_bytes = _workspace(ws, M, K, N, dev)
    if smooth is not None:
        _need(smooth, "smooth", torch.float32, (K,), dev)
        st = lib().wq_gemm_w8a8_smooth(_ptr(X), _ptr(smooth), _ptr(Wq), _ptr(Sw), _ptr(Y), _ptr(Xq),
                                       _ptr(Sx), _ptr(acc), _ptr(ws), ws_bytes, M, K, N, _stream(dev))
        _check("wq_gemm_w8a8_smooth", st)
        return Y, Xq, Sx, acc
    st = lib().wq_gemm_w8a8(_ptr(X), _ptr(Wq), _ptr(Sw), _ptr(Y), _ptr(Xq), _ptr(Sx), _ptr(acc),
                            _ptr(ws), ws_bytes, M, K, N, _stream(dev))
    _check("wq_gemm_w8a8", st)
    return Y, Xq, Sx, acc


def gemm_w8a8_noalloc(X, Wq, Sw, Y, Xq, Sx, acc=None):
    """wq_gemm_w8a8_noalloc: W8A8 into caller-given outputs, workspace held by the library.

    Every output tensor is passed in (nothing is allocated here either):
    Y bf16 [M,N], Xq int8 [M,K], Sx fp32 [M], acc int32 [M,N] or None.
    """
    M, K = X.shape
    N = Wq.shape[0]
    dev = X.device
    _need(X, "X", torch.float32, (M, K), dev)
    _need(Wq, "Wq", torch.int8, (N, K), dev)
    _need(Sw, "Sw", torch.float32, (N,), dev)
    _need(Y, "Y", torch.bfloat16, (M, N), dev)
    _need(Xq, "Xq", torch.int8, (M, K), dev)
    _need(Sx, "Sx", torch.float32, (M,), dev)
    if acc is not None:
        _need(acc, "acc", torch.int32, (M, N), dev)
    st = lib().wq_gemm_w8a8_noalloc(_ptr(X), _ptr(Wq), _ptr(Sw), _ptr(Y), _ptr(Xq), _ptr(Sx),
                                    _ptr(acc), M, K, N, _stream(dev))
    _check("wq_gemm_w8a8_noalloc", st)


def gemm_int8_mixed(X, W16, threshold=6.0, want_acc=False, Y=None, ws=None):
    """LLM.int8() decomposition of fp16 X [M, K] times the fp16 weight W16 [N, K].

    Returns ``(Y fp16 [M,N], Xq, Sx, Wq, Sw, colmax [K], outlier_mask [K/32],
    outlier_cols [K], n_outlier [1], acc | None)``, all on the device: the
    first ``n_outlier`` entries of ``outlier_cols`` list the outlier columns.
    Nothing is read back to the host, so the call can be captured into a
    graph.
    """
    M, K = X.shape
    N = W16.shape[0]
    dev = X.device
    _need(X, "X", torch.float16, (M, K), dev)
    _need(W16, "W16", torch.float16, (N, K), dev)
    Y = torch.empty((M, N), dtype=torch.float16, device=dev) if Y is None else Y
    _need(Y, "Y", torch.float16, (M, N), dev)
    Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    Sx = torch.empty(M, dtype=torch.float32, device=dev)
    Wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    Sw = torch.empty(N, dtype=torch.float32, device=dev)
    colmax = torch.empty(K, dtype=torch.float32, device=dev)
    mask = torch.empty((K + 31) // 32, dtype=torch.int32, device=dev)
    cols = torch.empty(K, dtype=torch.int32, device=dev)
    n_out = torch.empty(1, dtype=torch.int32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    ws, ws_bytes = _workspace(ws, M, K, N, dev)
    st = lib().wq_gemm_int8_mixed(_ptr(X), _ptr(W16), float(threshold), _ptr(Y), _ptr(Xq), _ptr(Sx),
                                  _ptr(Wq), _ptr(Sw), _ptr(colmax), _ptr(mask), _ptr(cols),
                                  _ptr(n_out), _ptr(acc), _ptr(ws), ws_bytes, M, K, N, _stream(dev))
    _check("wq_gemm_int8_mixed", st)
    return Y, Xq, Sx, Wq, Sw, colmax, mask, cols, n_out, acc


# ---------------------------------------------------------- measurement --

def calib_empty(sink, grid: int = 256, threads: int = 512):
    """One launch of an empty kernel (the dispatch floor); sink: int32 [1] on the device."""
    dev = sink.device
    _need(sink, "sink", torch.int32, (1,), dev)
    _check("wq_calib_empty", lib().wq_calib_empty(grid, threads, _ptr(sink), _stream(dev)))


def calib_stream_read(buf, sink):
    """One launch that only reads the bytes of ``buf`` once (the int8 GEMV's loads)."""
    dev = buf.device
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _need(sink, "sink", torch.int32, (1,), dev)
    nbytes = buf.numel() * buf.element_size()
    _check("wq_calib_stream_read",
           lib().wq_calib_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(dev)))
