"""C-ABI checks that need no GPU: the library loads, exports every function
``include/wq.h`` declares, rejects bad arguments on the host before any HIP
call, and its host-only act-order permutation is correct."""
import ctypes

import numpy as np
import pytest

wq = pytest.importorskip("weight_only_quantized_dequant_amd")

# Non-NULL, 16-byte-aligned dummy "device" addresses.  Every call below fails
# its host-side checks, so none of them is ever dereferenced or launched.
P = ctypes.c_void_p(1 << 20)
P_MIS = ctypes.c_void_p((1 << 20) + 2)


@pytest.fixture(scope="module")
def L():
    return wq.lib()


def test_exports_every_declared_symbol(L):
    names = wq.header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for st in range(7):
        assert L.wq_status_str(st)
    assert L.wq_status_str(99) == b"unknown status"
    assert L.wq_last_hip_error() == 0


def test_workspace_bytes_pure_and_valid(L):
    a = L.wq_workspace_bytes(wq.WQ_OP_Q8G, 1, 4096, 4096, 128)
    assert a > 0 and a == L.wq_workspace_bytes(wq.WQ_OP_Q8G, 1, 4096, 4096, 128)
    assert L.wq_workspace_bytes(wq.WQ_OP_Q3, 1, 4096, 11008, 0) > 0
    assert L.wq_workspace_bytes(wq.WQ_OP_Q4G, 8, 4096, 11008, 128) > 0
    # invalid shapes / ops -> 0
    assert L.wq_workspace_bytes(wq.WQ_OP_Q8G, 1, 4096, 4095, 128) == 0
    assert L.wq_workspace_bytes(wq.WQ_OP_Q3, 1, 100, 64, 0) == 0
    assert L.wq_workspace_bytes(7, 1, 4096, 4096, 128) == 0


def test_q3_validation(L):
    f = L.wq_matvec_q3
    ws = 1 << 20
    assert f(None, P, P, P, P, 64, 64, 0, P, ws, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, P, P, 64, 64, 5, P, ws, None) == wq.WQ_ERR_DTYPE
    assert f(P, P, P, P, P, 48, 64, 0, P, ws, None) == wq.WQ_ERR_SHAPE   # K % 32
    assert f(P, P, P, P, P, 64, 62, 0, P, ws, None) == wq.WQ_ERR_SHAPE   # N % 4
    assert f(P_MIS, P, P, P, P, 64, 64, 0, P, ws, None) == wq.WQ_ERR_ALIGN
    assert f(P, P, P, P, P, 64, 64, 1, None, 0, None) in (wq.WQ_ERR_WORKSPACE,)
    need = L.wq_workspace_bytes(wq.WQ_OP_Q3, 1, 4096, 4096, 0)
    assert f(P, P, P, P, P, 4096, 4096, 1, P, need - 1, None) == wq.WQ_ERR_WORKSPACE


def test_q8_validation(L):
    f = L.wq_gemm_q8_group
    ws = 1 << 24
    assert f(P, None, P, P, 1, 4096, 4096, 128, P, ws, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, P, 0, 4096, 4096, 128, P, ws, None) == wq.WQ_ERR_SHAPE    # M
    assert f(P, P, P, P, 1, 4096, 4104, 128, P, ws, None) == wq.WQ_ERR_SHAPE    # N % 16
    assert f(P, P, P, P, 1, 4096, 4096, 96, P, ws, None) == wq.WQ_ERR_SHAPE     # K % G
    assert f(P, P, P, P, 1, 4096, 4096, 48, P, ws, None) == wq.WQ_ERR_SHAPE     # G % 32
    assert f(P, P_MIS, P, P, 1, 4096, 4096, 128, P, ws, None) == wq.WQ_ERR_ALIGN
    need = L.wq_workspace_bytes(wq.WQ_OP_Q8G, 1, 4096, 4096, 128)
    assert f(P, P, P, P, 1, 4096, 4096, 128, P, need - 16, None) == wq.WQ_ERR_WORKSPACE
    assert f(P, P, P, P, 1, 4096, 4096, 128, P_MIS, need, None) == wq.WQ_ERR_ALIGN


def test_q4_validation(L):
    f = L.wq_gemm_q4_group
    ws = 1 << 24
    assert f(P, P, None, None, P, 1, 4096, 11008, 128, P, ws, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, None, P, 1, 4096, 11006, 128, P, ws, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, None, P, 1, 4000, 11008, 128, P, ws, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, None, P, 1, 4096, 11008, 16, P, ws, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, None, P, 1, 4096, 11008, 128, None, 0, None) == wq.WQ_ERR_WORKSPACE
    g = L.wq_q4_prepack
    assert g(P, P, P, 12, 16, None) == wq.WQ_ERR_SHAPE
    assert g(P, P, P, 64, 16, None) == wq.WQ_ERR_SHAPE   # in == out (overlap)
    assert g(P, None, ctypes.c_void_p(1 << 30), 64, 16, None) == wq.WQ_ERR_NULL


def test_w8a8_validation(L):
    f = L.wq_gemm_w8a8
    assert f(P, P, P, P, P, None, None, 256, 8192, 8192, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, P, P, P, None, 256, 8190, 8192, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, P, P, None, 256, 8192, 8200, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, P, P, None, 0, 8192, 8192, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, P, P, None, 1, 1 << 20, 64, None) == wq.WQ_ERR_SHAPE  # int32 range
    assert f(P, P_MIS, P, P, P, P, None, 256, 8192, 8192, None) == wq.WQ_ERR_ALIGN


def test_unpack_validation(L):
    assert L.wq_unpack_q3(P, P, 33, 64, None) == wq.WQ_ERR_SHAPE
    assert L.wq_unpack_q4(P, None, P, 12, 64, None) == wq.WQ_ERR_SHAPE
    assert L.wq_unpack_q4(None, None, P, 64, 64, None) == wq.WQ_ERR_NULL


def test_act_order_perm_host():
    rng = np.random.default_rng(5)
    K, G = 512, 128
    g_idx = rng.permutation(np.repeat(np.arange(K // G), G)).astype(np.int32)
    perm = wq.q4_act_order_perm(g_idx, K, G)
    assert sorted(perm.tolist()) == list(range(K))
    # rows [gG, gG+G) of the new order all belong to group g, in increasing k
    for g in range(K // G):
        seg = perm[g * G:(g + 1) * G]
        assert np.all(g_idx[seg] == g)
        assert np.all(np.diff(seg) > 0)
    assert np.array_equal(wq.q4_act_order_perm(None, K, G), np.arange(K))
    bad = g_idx.copy()
    bad[0], bad[1] = 0, 0
    if np.bincount(bad, minlength=K // G).max() != G or np.bincount(bad).min() != G:
        with pytest.raises(wq.WQError):
            wq.q4_act_order_perm(bad, K, G)
    with pytest.raises(wq.WQError):
        wq.q4_act_order_perm(np.full(K, 9, np.int32), K, G)
