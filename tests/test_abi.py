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


def test_packed_bytes_pure_and_valid(L):
    a = L.wq_packed_bytes(wq.WQ_OP_Q8G, 4096, 4096, 128)
    assert a == 4096 * 4096 and a == L.wq_packed_bytes(wq.WQ_OP_Q8G, 4096, 4096, 0)
    # int8 column pairs: exactly the stored weight's K * N bytes at any legal shape.
    for K, N in ((32, 16), (96, 48), (4224, 272), (11008, 4096), (8192, 11008)):
        assert L.wq_packed_bytes(wq.WQ_OP_Q8G, K, N, 32) == K * N
    # the configured shapes re-lay out without padding
    assert L.wq_packed_bytes(wq.WQ_OP_Q3, 4096, 11008, 0) == 4096 // 32 * 3 * 11008 * 4
    assert L.wq_packed_bytes(wq.WQ_OP_Q3, 11008, 4096, 0) >= 11008 // 32 * 3 * 4096 * 4
    # 4-bit: the codes plus the uint16 row table
    # blocks, the inverse row table, the forward row table (K rounded up to 128)
    assert L.wq_packed_bytes(wq.WQ_OP_Q4G, 4096, 11008, 128) == 4096 // 8 * 11008 * 4 + 4096 * 2 * 2
    assert L.wq_packed_bytes(wq.WQ_OP_Q4G, 4160, 64, 32) == 33 * 4 * 1024 + 4160 * 2 + 4224 * 2
    # invalid shapes / ops -> 0
    assert L.wq_packed_bytes(wq.WQ_OP_Q8G, 4096, 4095, 128) == 0
    assert L.wq_packed_bytes(wq.WQ_OP_Q3, 100, 64, 0) == 0
    assert L.wq_packed_bytes(wq.WQ_OP_Q4G, 4096, 11008, 96) == 0   # G not a power of two
    assert L.wq_packed_bytes(7, 4096, 4096, 128) == 0


def test_q3_validation(L):
    f = L.wq_matvec_q3
    assert f(None, P, P, P, P, 64, 64, 0, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, P, P, 64, 64, 5, None) == wq.WQ_ERR_DTYPE
    assert f(P, P, P, P, P, 48, 64, 0, None) == wq.WQ_ERR_SHAPE   # K % 32
    assert f(P, P, P, P, P, 64, 62, 0, None) == wq.WQ_ERR_SHAPE   # N % 4
    assert f(P, P, P, P, P, 32768 + 32, 64, 1, None) == wq.WQ_ERR_SHAPE  # LDS bound
    assert f(P_MIS, P, P, P, P, 64, 64, 0, None) == wq.WQ_ERR_ALIGN
    assert f(P, P_MIS, P, P, P, 64, 64, 0, None) == wq.WQ_ERR_ALIGN
    assert L.wq_prepack_q3(P, None, 64, 64, None) == wq.WQ_ERR_NULL
    assert L.wq_prepack_q3(P, P, 64, 66, None) == wq.WQ_ERR_SHAPE


def test_dequant_q8_validation(L):
    f = L.wq_dequant_q8_group
    assert f(None, P, P, 4096, 4096, 128, wq.WQ_F32, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, 4096, 4104, 128, wq.WQ_F32, None) == wq.WQ_ERR_SHAPE    # N % 16
    assert f(P, P, P, 4096, 4096, 96, wq.WQ_F16, None) == wq.WQ_ERR_SHAPE     # K % G
    assert f(P, P, P, 4096, 4096, 128, 7, None) == wq.WQ_ERR_SHAPE            # dtype
    assert f(P, P, P, 32768, 32768, 128, wq.WQ_F32, None) == wq.WQ_ERR_SHAPE  # W >= 2^31 bytes
    assert f(P, P, P_MIS, 4096, 4096, 128, wq.WQ_F16, None) == wq.WQ_ERR_ALIGN


def test_q8_validation(L):
    f = lambda *a: L.wq_gemm_q8_group(*a[:8], None, 0, a[8])        # no workspace
    assert f(P, None, P, P, 1, 4096, 4096, 128, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, P, 0, 4096, 4096, 128, None) == wq.WQ_ERR_SHAPE    # M
    assert f(P, P, P, P, 1, 4096, 4104, 128, None) == wq.WQ_ERR_SHAPE    # N % 16
    assert f(P, P, P, P, 1, 4096, 4096, 96, None) == wq.WQ_ERR_SHAPE     # K % G
    assert f(P, P, P, P, 1, 4096, 4096, 48, None) == wq.WQ_ERR_SHAPE     # G % 32
    assert f(P, P_MIS, P, P, 1, 4096, 4096, 128, None) == wq.WQ_ERR_ALIGN
    assert f(P, P, P, P_MIS, 8, 4096, 4096, 128, None) == wq.WQ_ERR_ALIGN    # Y: 8-byte stores
    # above 32 rows the tiled path splits K: S slices of M x N fp32 partials
    need = L.wq_workspace_bytes(wq.WQ_OP_Q8G, 33, 4096, 4096)
    assert need == 8 * 33 * 4096 * 4
    assert L.wq_workspace_bytes(wq.WQ_OP_Q8G, 32, 4096, 4096) == 0     # one streaming pass
    assert L.wq_workspace_bytes(wq.WQ_OP_Q8G, 17, 4096, 4096) == 0
    assert L.wq_workspace_bytes(wq.WQ_OP_Q8G, 64, 4096, 4096) == 8 * 64 * 4096 * 4
    assert L.wq_workspace_bytes(wq.WQ_OP_Q8G, 256, 4096, 4096) == 2 * 256 * 4096 * 4
    assert L.wq_workspace_bytes(wq.WQ_OP_Q8G, 512, 4096, 4096) == 0    # 512 tiles fill the GPU
    assert L.wq_workspace_bytes(wq.WQ_OP_Q8G, 33, 4160, 4096) == 0     # K not whole slices
    g8 = L.wq_gemm_q8_group
    assert g8(P, P, P, P, 33, 4096, 4096, 128, None, need, None) == wq.WQ_ERR_WORKSPACE
    assert g8(P, P, P, P, 33, 4096, 4096, 128, P, need - 16, None) == wq.WQ_ERR_WORKSPACE
    assert g8(P, P, P, P, 33, 4096, 4096, 128, P_MIS, need, None) == wq.WQ_ERR_ALIGN
    # groups of 32 run as streaming passes at any M: no workspace
    assert f(P, P, P, P_MIS, 16, 4096, 4096, 32, None) == wq.WQ_ERR_ALIGN  # (reaches the Y check)
    assert L.wq_prepack_q8(P, P, 4096, 4100, None) == wq.WQ_ERR_SHAPE
    assert L.wq_prepack_q8(P_MIS, P, 4096, 4096, None) == wq.WQ_ERR_ALIGN


def test_q4_validation(L):
    f = lambda *a: L.wq_gemm_q4_group(*a[:8], None, 0, a[8])        # no workspace
    assert f(P, P, None, P, 1, 4096, 11008, 128, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, P, 1, 4096, 11006, 128, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, 1, 4000, 11008, 128, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, 1, 4096, 11008, 16, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, 0, 4096, 11008, 128, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, 1, 32768 + 128, 64, 128, None) == wq.WQ_ERR_SHAPE   # K bound
    assert f(P, P_MIS, P, P, 1, 4096, 11008, 128, None) == wq.WQ_ERR_ALIGN
    # above 4 rows: X in the packed row order (rows rounded up to 16, K to 128, fp16)
    q4ws = lambda Mp, Kp: Mp * Kp * 2
    need = L.wq_workspace_bytes(wq.WQ_OP_Q4G, 64, 4096, 11008)
    assert need == q4ws(64, 4096)
    assert L.wq_workspace_bytes(wq.WQ_OP_Q4G, 4, 4096, 11008) == 0
    assert L.wq_workspace_bytes(wq.WQ_OP_Q4G, 5, 4096, 11008) == q4ws(16, 4096)
    assert L.wq_workspace_bytes(wq.WQ_OP_Q4G, 9, 4160, 11008) == q4ws(16, 4224)
    g4 = L.wq_gemm_q4_group
    assert g4(P, P, P, P, 64, 4096, 11008, 128, None, need, None) == wq.WQ_ERR_WORKSPACE
    assert g4(P, P, P, P, 64, 4096, 11008, 128, P, need - 2, None) == wq.WQ_ERR_WORKSPACE
    assert g4(P, P, P, P, 64, 4096, 11008, 128, P_MIS, need, None) == wq.WQ_ERR_ALIGN
    z = lambda *a: L.wq_gemm_q4_group_zp(*a[:9], None, 0, a[9])
    assert z(P, P, P, None, P, 1, 4096, 11008, 128, None) == wq.WQ_ERR_NULL      # zeros
    assert z(P, P, P, P, P, 1, 4096, 11006, 128, None) == wq.WQ_ERR_SHAPE
    assert z(P, P, P, P_MIS, P, 1, 4096, 11008, 128, None) == wq.WQ_ERR_ALIGN
    assert z(P, P, P, P, P, 16, 4096, 11008, 128, None) == wq.WQ_ERR_WORKSPACE
    g = L.wq_prepack_q4
    assert g(P, None, P, 12, 16, 32, None) == wq.WQ_ERR_SHAPE
    assert g(P, None, None, 64, 16, 32, None) == wq.WQ_ERR_NULL


def test_q2_validation(L):
    assert L.wq_packed_bytes(wq.WQ_OP_Q2G, 4096, 11008, 128) == 4096 // 16 * 11008 * 4 + 4096 * 2
    assert L.wq_packed_bytes(wq.WQ_OP_Q2G, 4096, 11008, 96) == 0
    f = L.wq_gemm_q2_group_zp
    assert f(P, P, P, None, P, 1, 4096, 11008, 128, None) == wq.WQ_ERR_NULL      # zeros
    assert f(P, P, P, P, P, 1, 4096, 11006, 128, None) == wq.WQ_ERR_SHAPE       # N % 4
    assert f(P, P, P, P, P, 1, 4000, 11008, 128, None) == wq.WQ_ERR_SHAPE       # K % G
    assert f(P, P, P, P, P, 1, 4096, 11008, 16, None) == wq.WQ_ERR_SHAPE        # G >= 32
    assert f(P, P, P, P, P, 0, 4096, 11008, 128, None) == wq.WQ_ERR_SHAPE       # M
    assert f(P, P, P, P, P, 1, 32768 + 128, 64, 128, None) == wq.WQ_ERR_SHAPE   # K bound
    assert f(P, P, P, P_MIS, P, 1, 4096, 11008, 128, None) == wq.WQ_ERR_ALIGN
    assert L.wq_prepack_q2(P, None, None, 64, 16, 32, None) == wq.WQ_ERR_NULL
    assert L.wq_prepack_q2(P, None, P, 48, 16, 32, None) == wq.WQ_ERR_SHAPE
    assert L.wq_unpack_q2(None, None, P, 64, 64, 32, None) == wq.WQ_ERR_NULL


def test_w8a8_validation(L):
    f = L.wq_gemm_w8a8
    WS = 64 << 20
    #        X  Wq Sw Y  Xq Sx acc  ws  bytes M    K     N
    assert f(P, P, P, P, P, None, None, P, WS, 256, 8192, 8192, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, P, P, P, None, P, WS, 256, 8190, 8192, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, P, P, None, P, WS, 256, 8192, 8200, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, P, P, None, P, WS, 0, 8192, 8192, None) == wq.WQ_ERR_SHAPE
    assert f(P, P, P, P, P, P, None, P, WS, 1, 1 << 20, 64, None) == wq.WQ_ERR_SHAPE  # int32 range
    assert f(P, P_MIS, P, P, P, P, None, P, WS, 256, 8192, 8192, None) == wq.WQ_ERR_ALIGN
    assert f(P, P, P, P_MIS, P, P, None, P, WS, 256, 8192, 8192, None) == wq.WQ_ERR_ALIGN  # Y
    assert f(P, P, P_MIS, P, P, P, None, P, WS, 256, 8192, 8192, None) == wq.WQ_ERR_ALIGN  # Sw
    assert f(P, P, P, P, P, P, P_MIS, P, WS, 256, 8192, 8192, None) == wq.WQ_ERR_ALIGN     # acc_out
    # the workspace: missing, too small, misaligned
    need = L.wq_workspace_bytes(wq.WQ_OP_W8A8, 256, 8192, 8192)
    assert need == 2 * 256 * 8192 * 4                                   # two K slices
    assert f(P, P, P, P, P, P, None, None, need, 256, 8192, 8192, None) == wq.WQ_ERR_WORKSPACE
    assert f(P, P, P, P, P, P, None, P, need - 16, 256, 8192, 8192, None) == wq.WQ_ERR_WORKSPACE
    assert f(P, P, P, P, P, P, None, P_MIS, need, 256, 8192, 8192, None) == wq.WQ_ERR_ALIGN
    assert L.wq_status_str(wq.WQ_ERR_WORKSPACE).startswith(b"workspace")


def test_w8a8_noalloc_validation(L):
    f = L.wq_gemm_w8a8_noalloc
    assert f(P, P, P, P, P, None, None, 256, 8192, 8192, None) == wq.WQ_ERR_NULL
    assert f(P, P, P, P, P, P, None, 256, 8190, 8192, None) == wq.WQ_ERR_SHAPE
    assert f(P, P_MIS, P, P, P, P, None, 256, 8192, 8192, None) == wq.WQ_ERR_ALIGN
    # 256 x 8704 with two K slices needs 17 MiB of partials: beyond the 16 MiB array
    assert f(P, P, P, P, P, P, None, 256, 8192, 8704, None) == wq.WQ_ERR_WORKSPACE


def test_workspace_bytes(L):
    w = lambda M, K, N, op=wq.WQ_OP_W8A8: L.wq_workspace_bytes(op, M, K, N)
    assert w(512, 8192, 8192) == 0                   # 4 x 64 output tiles fill the GPU: no split
    assert w(256, 8192, 8192) == 2 * 256 * 8192 * 4  # 128 tiles: two K slices
    assert w(64, 8192, 4096) == 8 * 64 * 4096 * 4    # 32 tiles: eight K slices
    assert w(1, 64, 16) == 0                         # a single stage of K: nothing to split
    assert w(256, 8190, 8192) == 0                   # invalid shape
    for op in (wq.WQ_OP_Q3, wq.WQ_OP_Q8G, wq.WQ_OP_Q2G):
        assert w(256, 8192, 8192, op) == 0           # these weight-only products need none
    assert w(256, 8192, 8192, wq.WQ_OP_Q4G) == 256 * 8192 * 2   # 4-bit: X in the packed row order
    f3 = lambda *a: L.wq_gemm_int8_mixed(*a[:13], P, 64 << 20, *a[13:])
    c6 = ctypes.c_float(6.0)
    #      X  W  thr Y  Xq Sx Wq Sw cm mk cols nout acc (ws, bytes)
    assert f3(P, P, c6, P, P, P, P, P, P, P, P, None, None, 64, 1024, 64, None) == wq.WQ_ERR_NULL  # n_outlier
    assert f3(P, None, c6, P, P, P, P, P, P, P, P, P, None, 64, 1024, 64, None) == wq.WQ_ERR_NULL  # W
    assert f3(P, P, c6, P, P, P, None, P, P, P, P, P, None, 64, 1024, 64, None) == wq.WQ_ERR_NULL  # Wq
    assert f3(P, P, c6, P, P, P, P, P, P, None, P, P, None, 64, 1024, 64, None) == wq.WQ_ERR_NULL  # mask
    assert f3(P, P, c6, P, P, P, P, P, P, P, P, P, None, 64, 1000, 64, None) == wq.WQ_ERR_SHAPE
    assert f3(P, P, c6, P, P, P, P, P, P, P, P, P, None, 64, 1024, 60, None) == wq.WQ_ERR_SHAPE
    assert f3(P, P, ctypes.c_float(float("nan")), P, P, P, P, P, P, P, P, P, None, 64, 1024, 64,
              None) == wq.WQ_ERR_SHAPE
    assert f3(P_MIS, P, c6, P, P, P, P, P, P, P, P, P, None, 64, 1024, 64, None) == wq.WQ_ERR_ALIGN
    assert f3(P, P_MIS, c6, P, P, P, P, P, P, P, P, P, None, 64, 1024, 64, None) == wq.WQ_ERR_ALIGN
    assert f3(P, P, c6, P, P, P, P, P, P, P_MIS, P, P, None, 64, 1024, 64, None) == wq.WQ_ERR_ALIGN
    f2 = L.wq_gemm_w8a8_smooth
    assert f2(P, None, P, P, P, P, P, None, P, 1 << 20, 64, 1024, 64, None) == wq.WQ_ERR_NULL    # smooth
    assert f2(P, P_MIS, P, P, P, P, P, None, P, 1 << 20, 64, 1024, 64, None) == wq.WQ_ERR_ALIGN
    assert f2(P, P, P, P, P, P, P, None, P, 1 << 20, 64, 1000, 64, None) == wq.WQ_ERR_SHAPE


def test_unpack_validation(L):
    assert L.wq_unpack_q3(P, P, 33, 64, None) == wq.WQ_ERR_SHAPE
    assert L.wq_unpack_q8(P, P, 64, 60, None) == wq.WQ_ERR_SHAPE
    assert L.wq_unpack_q4(P, None, P, 12, 64, 32, None) == wq.WQ_ERR_SHAPE
    assert L.wq_unpack_q4(None, None, P, 64, 64, 32, None) == wq.WQ_ERR_NULL


def test_act_order_perm_host():
    rng = np.random.default_rng(5)
    K, G = 512, 128
    g_idx = rng.permutation(np.repeat(np.arange(K // G), G)).astype(np.int32)
    perm, inv = wq.q4_act_order_perm(g_idx, K, G)
    assert sorted(perm.tolist()) == list(range(K))
    assert np.array_equal(inv[perm], np.arange(K))
    # rows [gG, gG+G) of the new order all belong to group g, in increasing k
    for g in range(K // G):
        seg = perm[g * G:(g + 1) * G]
        assert np.all(g_idx[seg] == g)
        assert np.all(np.diff(seg) > 0)
    p0, i0 = wq.q4_act_order_perm(None, K, G)
    assert np.array_equal(p0, np.arange(K)) and np.array_equal(i0, np.arange(K))
    bad = g_idx.copy()
    bad[np.nonzero(bad == 1)[0][0]] = 0      # group 0 gets G+1 rows, group 1 G-1
    with pytest.raises(wq.WQError):
        wq.q4_act_order_perm(bad, K, G)
    with pytest.raises(wq.WQError):
        wq.q4_act_order_perm(np.full(K, 9, np.int32), K, G)


def test_calibration_validation(L):
    assert L.wq_calib_empty(256, 512, None, None) == wq.WQ_ERR_NULL
    assert L.wq_calib_empty(0, 512, P, None) == wq.WQ_ERR_SHAPE
    assert L.wq_calib_empty(256, 2048, P, None) == wq.WQ_ERR_SHAPE
    f = L.wq_calib_stream_read
    assert f(None, 1 << 20, P, None) == wq.WQ_ERR_NULL
    assert f(P, 1 << 20, None, None) == wq.WQ_ERR_NULL
    assert f(P, 1000, P, None) == wq.WQ_ERR_SHAPE          # bytes % 16
    assert f(P, 0, P, None) == wq.WQ_ERR_SHAPE
    assert f(P, 1 << 31, P, None) == wq.WQ_ERR_SHAPE        # 32-bit buffer offsets
    assert f(P_MIS, 1 << 20, P, None) == wq.WQ_ERR_ALIGN
