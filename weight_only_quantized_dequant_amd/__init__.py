"""Python binding of libwq.so: fused low-bit dequantize-and-multiply on MI355X.

Argument marshalling only.  Every step of every product runs in the HIP
kernels of libwq.so; torch supplies device memory and the current stream.
There is no fallback: without the built library every call raises.

Entry points (same names as the C ABI in ``include/wq.h``):

* ``matvec_q3(x, qweight, scales, zeros)``            -> y
* ``gemm_q8_group(X, qweight, scales, group_size)``   -> Y
* ``q4_act_order_perm(g_idx, K, group_size)``         -> perm (host, int32)
* ``q4_prepack(qweight, perm)``                       -> prepacked qweight
* ``gemm_q4_group(X, qweight, scales, perm, group_size)`` -> Y
* ``gemm_w8a8(X, Wq, Sw, want_acc=False)``            -> (Y bf16, Xq, Sx, acc|None)
* ``unpack_q3(qweight, K)`` / ``unpack_q4(qweight, K, perm=None)`` -> int8 codes
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

WQ_OK, WQ_ERR_NULL, WQ_ERR_SHAPE, WQ_ERR_ALIGN, WQ_ERR_DTYPE, WQ_ERR_WORKSPACE, WQ_ERR_HIP = range(7)
WQ_F32, WQ_F16 = 0, 1
WQ_OP_Q3, WQ_OP_Q4G, WQ_OP_Q8G = 0, 1, 2

_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGNATURES = {
    "wq_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "wq_matvec_q3": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]),
    "wq_gemm_q8_group": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "wq_q4_act_order_perm": (_i, [_vp, _i, _i, _vp]),
    "wq_q4_prepack": (_i, [_vp, _vp, _vp, _i, _i, _vp]),
    "wq_gemm_q4_group": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "wq_gemm_w8a8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp]),
    "wq_unpack_q3": (_i, [_vp, _vp, _i, _i, _vp]),
    "wq_unpack_q4": (_i, [_vp, _vp, _vp, _i, _i, _vp]),
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


# Per-(device, stream) workspaces: zero-filled once, left zeroed by every call.
_workspaces: dict = {}


def workspace(op: int, M: int, K: int, N: int, G: int, device: torch.device) -> torch.Tensor:
    need = int(lib().wq_workspace_bytes(op, M, K, N, G))
    if need == 0:
        _check("wq_workspace_bytes", WQ_ERR_SHAPE)
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1 << 16), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def workspace_bytes(op: int, M: int, K: int, N: int, G: int) -> int:
    return int(lib().wq_workspace_bytes(op, M, K, N, G))


# ----------------------------------------------------------------- 3-bit --

def matvec_q3(x, qweight, scales, zeros, y=None):
    """y = x . (scale * q - zero) for a 3-bit packed weight; fp32 or fp16."""
    K = x.shape[0]
    N = qweight.shape[1]
    dt = x.dtype
    if dt not in (torch.float32, torch.float16):
        raise TypeError("x must be float32 or float16")
    dev = x.device
    _need(x, "x", dt, (K,), dev)
    _need(qweight, "qweight", torch.int32, (3 * K // 32, N), dev)
    _need(scales, "scales", dt, (N,), dev)
    _need(zeros, "zeros", dt, (N,), dev)
    if y is None:
        y = torch.empty(N, dtype=dt, device=dev)
    _need(y, "y", dt, (N,), dev)
    ws = workspace(WQ_OP_Q3, 1, K, N, 0, dev)
    st = lib().wq_matvec_q3(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(y), K, N,
                            WQ_F16 if dt == torch.float16 else WQ_F32, _ptr(ws), ws.numel(),
                            _stream(dev))
    _check("wq_matvec_q3", st)
    return y


# ------------------------------------------------------------------ int8 --

def gemm_q8_group(X, qweight, scales, group_size=128, Y=None):
    """Y = X . (scale[k // G] * q) for a group-wise int8 weight [K, N]."""
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    M, K = X2.shape
    N = qweight.shape[1]
    dev = X.device
    _need(X2, "X", torch.float16, (M, K), dev)
    _need(qweight, "qweight", torch.int8, (K, N), dev)
    _need(scales, "scales", torch.float32, (K // group_size, N), dev)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(Y, "Y", torch.float16, (M, N), dev)
    ws = workspace(WQ_OP_Q8G, M, K, N, group_size, dev)
    st = lib().wq_gemm_q8_group(_ptr(X2), _ptr(qweight), _ptr(scales), _ptr(Y), M, K, N,
                                group_size, _ptr(ws), ws.numel(), _stream(dev))
    _check("wq_gemm_q8_group", st)
    return Y.reshape(N) if squeeze else Y


# ----------------------------------------------------------------- 4-bit --

def q4_act_order_perm(g_idx, K: int, group_size: int = 128) -> np.ndarray:
    """Host: rows listed group by group (stable); ``g_idx=None`` is the identity."""
    perm = np.empty(K, dtype=np.int32)
    if g_idx is None:
        st = lib().wq_q4_act_order_perm(None, K, group_size, perm.ctypes.data_as(ctypes.c_void_p))
    else:
        g = np.ascontiguousarray(np.asarray(g_idx.cpu() if isinstance(g_idx, torch.Tensor) else g_idx,
                                            dtype=np.int32))
        if g.shape != (K,):
            raise ValueError(f"g_idx must have shape ({K},)")
        st = lib().wq_q4_act_order_perm(g.ctypes.data_as(ctypes.c_void_p), K, group_size,
                                        perm.ctypes.data_as(ctypes.c_void_p))
    _check("wq_q4_act_order_perm", st)
    return perm


def q4_prepack(qweight, perm):
    """Device: reorder the rows of a 4-bit weight into ``perm`` order."""
    R, N = qweight.shape
    K = 8 * R
    dev = qweight.device
    _need(qweight, "qweight", torch.int32, (R, N), dev)
    _need(perm, "perm", torch.int32, (K,), dev)
    out = torch.empty_like(qweight)
    st = lib().wq_q4_prepack(_ptr(qweight), _ptr(perm), _ptr(out), K, N, _stream(dev))
    _check("wq_q4_prepack", st)
    return out


def prepare_q4(qweight, g_idx, group_size=128):
    """Act-order preparation: returns ``(qweight_prepacked, perm_device)``."""
    K = 8 * qweight.shape[0]
    perm = torch.from_numpy(q4_act_order_perm(g_idx, K, group_size)).to(qweight.device)
    return q4_prepack(qweight, perm), perm


def gemm_q4_group(X, qweight, scales, perm=None, group_size=128, Y=None):
    """Y[m, n] = sum_i X[m, perm[i]] * scale[i // G, n] * q'[i, n] (prepacked q')."""
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    M, K = X2.shape
    N = qweight.shape[1]
    dev = X.device
    _need(X2, "X", torch.float16, (M, K), dev)
    _need(qweight, "qweight", torch.int32, (K // 8, N), dev)
    _need(scales, "scales", torch.float16, (K // group_size, N), dev)
    if perm is not None:
        _need(perm, "perm", torch.int32, (K,), dev)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(Y, "Y", torch.float16, (M, N), dev)
    ws = workspace(WQ_OP_Q4G, M, K, N, group_size, dev)
    st = lib().wq_gemm_q4_group(_ptr(X2), _ptr(qweight), _ptr(scales), _ptr(perm), _ptr(Y), M, K,
                                N, group_size, _ptr(ws), ws.numel(), _stream(dev))
    _check("wq_gemm_q4_group", st)
    return Y.reshape(N) if squeeze else Y


# ------------------------------------------------------------------ W8A8 --

def gemm_w8a8(X, Wq, Sw, want_acc=False, Y=None, Xq=None, Sx=None, acc=None):
    """Dynamic W8A8: returns ``(Y bf16 [M,N], Xq int8 [M,K], Sx fp32 [M], acc int32 | None)``."""
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
    st = lib().wq_gemm_w8a8(_ptr(X), _ptr(Wq), _ptr(Sw), _ptr(Y), _ptr(Xq), _ptr(Sx), _ptr(acc),
                            M, K, N, _stream(dev))
    _check("wq_gemm_w8a8", st)
    return Y, Xq, Sx, acc


# ---------------------------------------------------------------- unpack --

def unpack_q3(qweight, K: int):
    N = qweight.shape[1]
    dev = qweight.device
    _need(qweight, "qweight", torch.int32, (3 * K // 32, N), dev)
    codes = torch.empty((K, N), dtype=torch.int8, device=dev)
    _check("wq_unpack_q3", lib().wq_unpack_q3(_ptr(qweight), _ptr(codes), K, N, _stream(dev)))
    return codes


def unpack_q4(qweight, K: int, perm=None):
    N = qweight.shape[1]
    dev = qweight.device
    _need(qweight, "qweight", torch.int32, (K // 8, N), dev)
    if perm is not None:
        _need(perm, "perm", torch.int32, (K,), dev)
    codes = torch.empty((K, N), dtype=torch.int8, device=dev)
    _check("wq_unpack_q4", lib().wq_unpack_q4(_ptr(qweight), _ptr(perm), _ptr(codes), K, N,
                                              _stream(dev)))
    return codes
