"""Seeded synthetic inputs for the fused dequantize-and-multiply paths.

This module is shared by the tests, the benchmark and the smoke check, and by
both sides of every parity comparison (the CPU oracle and the HIP library).
It only *prepares inputs*: random draws, the offline weight quantisers that
turn an fp32 weight into stored codes plus scales (done once, before
inference, as the "Quantization CUDA" page (tom-jerr.github.io) describes in
"Dynamic Quantization": weights are quantised in preprocessing), and the
packers that write codes into their stored bit layout.  It holds none of the
arithmetic of the path itself: no unpacking, no dequantisation, no product,
no activation quantiser and no epilogue.

Stored layouts written here:

* 3-bit: int32 ``[3K/32, N]``; for column ``n`` and 32-row block ``b`` the
  words ``3b, 3b+1, 3b+2`` form a 96-bit little-endian value whose bits
  ``3i..3i+2`` hold the code of row ``32b + i``.
* 4-bit: int32 ``[K/8, N]``; nibble ``j`` (bits ``4j..4j+3``) of word ``r``
  holds row ``8r + j`` as the unsigned value ``q + 8``.
* int8: ``[K, N]`` (weight-only) or ``[N, K]`` (the W8A8 weight).

All draws use numpy's PCG64 (``numpy.random.default_rng``), in the order the
functions list them.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "pack_q3", "pack_q4", "gen_q3", "gen_q8_group", "gen_q4_group",
    "gen_w8a8", "gen_q4_zp", "gen_w8a8_smooth", "gen_int8_mixed", "SEEDS",
    "pack_q2", "gen_q2_zp",
]

# Seeds of the named workloads (the tests and the benchmark use these).
SEEDS = {
    "q3_f32_1024": 1000,
    "q8_group_4096": 1100,
    "q8_group_m512": 1500,       # M = 512, K = N = 4096 (the tiled matrix-core path)
    "q3_f16_4096x4096": 1200,
    "q3_f16_4096x11008": 1201,
    "q3_f16_11008x4096": 1202,
    "q4_group_actorder": 1300,   # weights; activations use 1300 + M
    "q4_zp": 1600,               # asymmetric 4-bit; activations use 1600 + M
    "w8a8_256x8192x8192": 1400,
    "w8a8_smooth": 1700,
    "int8_mixed": 1800,
    "q2_zp": 1900,               # asymmetric 2-bit; activations use 1900 + M
}


def pack_q3(codes: np.ndarray) -> np.ndarray:
    """Pack 3-bit codes ``[K, N]`` (values 0..7, K % 32 == 0) into int32 words."""
    codes = np.asarray(codes)
    K, N = codes.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if codes.min(initial=0) < 0 or codes.max(initial=0) > 7:
        raise ValueError("3-bit codes must lie in 0..7")
    c = codes.astype(np.uint64).reshape(K // 32, 32, N)
    words = np.zeros((K // 32, 3, N), dtype=np.uint64)
    mask32 = np.uint64(0xFFFFFFFF)
    for i in range(32):
        word, off = divmod(3 * i, 32)
        words[:, word, :] |= (c[:, i, :] << np.uint64(off)) & mask32
        if off > 29:  # the code runs past the top of this word
            words[:, word + 1, :] |= c[:, i, :] >> np.uint64(32 - off)
    return words.reshape(3 * (K // 32), N).astype(np.uint32).view(np.int32)


def pack_q4(u: np.ndarray) -> np.ndarray:
    """Pack unsigned 4-bit values ``[K, N]`` (0..15, K % 8 == 0) into int32 words."""
    u = np.asarray(u)
    K, N = u.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    if u.min(initial=0) < 0 or u.max(initial=0) > 15:
        raise ValueError("4-bit values must lie in 0..15")
    v = u.astype(np.uint32).reshape(K // 8, 8, N)
    words = np.zeros((K // 8, N), dtype=np.uint32)
    for j in range(8):
        words |= v[:, j, :] << np.uint32(4 * j)
    return words.view(np.int32)


def pack_q2(u: np.ndarray) -> np.ndarray:
    """Pack unsigned 2-bit values ``[K, N]`` (0..3, K % 16 == 0) into int32 words."""
    u = np.asarray(u)
    K, N = u.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    if u.min(initial=0) < 0 or u.max(initial=0) > 3:
        raise ValueError("2-bit values must lie in 0..3")
    v = u.astype(np.uint32).reshape(K // 16, 16, N)
    words = np.zeros((K // 16, N), dtype=np.uint32)
    for j in range(16):
        words |= v[:, j, :] << np.uint32(2 * j)
    return words.view(np.int32)


def _absmax_scale(w: np.ndarray, axis: int, qmax: float) -> np.ndarray:
    """fp32 ``max|w| / qmax`` along ``axis``; used by the offline weight quantisers."""
    a = np.max(np.abs(w), axis=axis).astype(np.float32)
    return (a / np.float32(qmax)).astype(np.float32)


def _quantise(w32: np.ndarray, s32: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Round-half-even of ``w / s`` in fp32, clamped to [lo, hi]; ``s == 0`` gives 0."""
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(w32 / s32)
    r = np.where(s32 == 0, np.float32(0), r)
    return np.clip(r, lo, hi).astype(np.int64)


def gen_q3(K: int, N: int, seed: int, dtype: str = "f32") -> dict:
    """3-bit GPTQ-style matvec inputs.

    Draw order: codes ~ U{0..7} [K,N]; scale ~ U[0.005, 0.02) [N]; z ~ U{0..7} [N];
    x ~ N(0,1) [K].  ``zero = scale * z`` (so ``w = scale*q - zero``).  With
    ``dtype="f16"`` the scale is rounded to fp16 first and
    ``zero = fp16(fp32(scale) * z)``; x is rounded to fp16.
    """
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 8, size=(K, N))
    if dtype == "f32":
        scale = rng.uniform(0.005, 0.02, size=N).astype(np.float32)
        z = rng.integers(0, 8, size=N)
        zero = (scale * z.astype(np.float32)).astype(np.float32)
        x = rng.standard_normal(K).astype(np.float32)
    elif dtype == "f16":
        scale = rng.uniform(0.005, 0.02, size=N).astype(np.float16)
        z = rng.integers(0, 8, size=N)
        zero = (scale.astype(np.float32) * z.astype(np.float32)).astype(np.float16)
        x = rng.standard_normal(K).astype(np.float16)
    else:
        raise ValueError(dtype)
    return {"x": x, "qweight": pack_q3(codes), "scales": scale, "zeros": zero,
            "codes": codes, "K": K, "N": N, "dtype": dtype}


def gen_q8_group(M: int, K: int, N: int, G: int, seed: int) -> dict:
    """Group-wise symmetric int8 weight-only inputs.

    Draw order: W ~ N(0, 0.02) fp32 [K,N]; then x ~ N(0,1) fp16 [M,K].
    Scale per (group, column) = fp32 absmax/127, stored fp32 ``[K/G, N]``;
    ``q = clip(rint(W/scale), -127, 127)`` stored int8 ``[K, N]``.
    """
    if K % G:
        raise ValueError("K must be a multiple of G")
    rng = np.random.default_rng(seed)
    W = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    Wg = W.reshape(K // G, G, N)
    scales = _absmax_scale(Wg, axis=1, qmax=127.0)          # [K/G, N]
    q = _quantise(Wg, scales[:, None, :], -127, 127).reshape(K, N).astype(np.int8)
    X = rng.standard_normal((M, K)).astype(np.float16)
    return {"X": X, "q": q, "scales": scales, "M": M, "K": K, "N": N, "G": G}


def gen_q4_group(M: int, K: int, N: int, G: int, seed: int, act_order: bool = True,
                 x_seed: int | None = None) -> dict:
    """4-bit symmetric group-wise inputs, optionally with an act-order ``g_idx``.

    Draw order (weight rng ``seed``): W ~ N(0, 0.02) fp32 [K,N]; then, with
    act-order, ``g_idx`` = a random permutation of ``repeat(arange(K/G), G)``
    (every group owns exactly G rows, scattered over K); without it
    ``g_idx[k] = k // G``.  Per (group, column) the fp16 scale is
    ``fp16(absmax/7)`` over the group's rows and
    ``q = clip(rint(W / fp32(scale[g_idx[k]])), -8, 7)``.  X ~ N(0,1) fp16
    [M,K] from rng ``x_seed`` (default ``seed + M``).
    """
    if K % G or K % 8:
        raise ValueError("K must be a multiple of G and of 8")
    rng = np.random.default_rng(seed)
    W = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    ng = K // G
    if act_order:
        g_idx = rng.permutation(np.repeat(np.arange(ng), G)).astype(np.int32)
    else:
        g_idx = (np.arange(K) // G).astype(np.int32)
    absmax = np.zeros((ng, N), dtype=np.float32)
    for g in range(ng):
        absmax[g] = np.max(np.abs(W[g_idx == g]), axis=0)
    scales = (absmax / np.float32(7.0)).astype(np.float16)      # [K/G, N]
    s_row = scales.astype(np.float32)[g_idx]                      # [K, N]
    q = _quantise(W, s_row, -8, 7)
    qweight = pack_q4(q + 8)
    xr = np.random.default_rng(seed + M if x_seed is None else x_seed)
    X = xr.standard_normal((M, K)).astype(np.float16)
    return {"X": X, "qweight": qweight, "scales": scales, "g_idx": g_idx,
            "codes": q, "M": M, "K": K, "N": N, "G": G}


def gen_q4_zp(M: int, K: int, N: int, G: int, seed: int, act_order: bool = False,
              x_seed: int | None = None) -> dict:
    """Asymmetric (AWQ-style) 4-bit group-wise inputs: unsigned values, a zero
    point and a scale per (group, column).

    Draw order (weight rng ``seed``): W ~ N(0, 0.02) fp32 [K,N]; then, with
    act-order, ``g_idx`` as in :func:`gen_q4_group` (else ``k // G``).  Per
    (group, column): ``scale = fp16((max - min) / 15)`` over the group's rows,
    ``zero = clip(rint(-min / fp32(scale)), 0, 15)`` (an integer, stored fp16)
    and ``u = clip(rint(W / fp32(scale)) + zero, 0, 15)``, packed as
    :func:`pack_q4`.  X ~ N(0,1) fp16 [M,K] from rng ``x_seed`` (default
    ``seed + M``).
    """
    if K % G or K % 8:
        raise ValueError("K must be a multiple of G and of 8")
    rng = np.random.default_rng(seed)
    W = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    ng = K // G
    if act_order:
        g_idx = rng.permutation(np.repeat(np.arange(ng), G)).astype(np.int32)
    else:
        g_idx = (np.arange(K) // G).astype(np.int32)
    wmin = np.zeros((ng, N), dtype=np.float32)
    wmax = np.zeros((ng, N), dtype=np.float32)
    for g in range(ng):
        wmin[g] = np.min(W[g_idx == g], axis=0)
        wmax[g] = np.max(W[g_idx == g], axis=0)
    scales = ((wmax - wmin) / np.float32(15.0)).astype(np.float16)   # [K/G, N]
    s32 = scales.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        z = np.where(s32 == 0, np.float32(0), np.rint(-wmin / s32))
    z = np.clip(z, 0, 15)
    zeros = z.astype(np.float16)
    u = np.clip(_quantise(W, s32[g_idx], -(1 << 20), 1 << 20) + z[g_idx].astype(np.int64), 0, 15)
    qweight = pack_q4(u)
    xr = np.random.default_rng(seed + M if x_seed is None else x_seed)
    X = xr.standard_normal((M, K)).astype(np.float16)
    return {"X": X, "qweight": qweight, "scales": scales, "zeros": zeros, "g_idx": g_idx,
            "u": u, "W": W, "M": M, "K": K, "N": N, "G": G}


def gen_q2_zp(M: int, K: int, N: int, G: int, seed: int, act_order: bool = False,
              x_seed: int | None = None) -> dict:
    """Asymmetric 2-bit group-wise inputs: unsigned values 0..3, a zero point
    and a scale per (group, column).

    Draw order (weight rng ``seed``): W ~ N(0, 0.02) fp32 [K,N]; then, with
    act-order, ``g_idx = permutation(repeat(arange(K/G), G))`` (else
    ``k // G``).  Per (group, column): ``scale = fp16((max - min) / 3)`` over
    the group's rows, ``zero = clip(rint(-min / fp32(scale)), 0, 3)`` (an
    integer, stored fp16) and ``u = clip(rint(W / fp32(scale)) + zero, 0, 3)``,
    packed as :func:`pack_q2`.  X ~ N(0,1) fp16 [M,K] from rng ``x_seed``
    (default ``seed + M``).
    """
    if K % G or K % 16:
        raise ValueError("K must be a multiple of G and of 16")
    rng = np.random.default_rng(seed)
    W = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    ng = K // G
    if act_order:
        g_idx = rng.permutation(np.repeat(np.arange(ng), G)).astype(np.int32)
    else:
        g_idx = (np.arange(K) // G).astype(np.int32)
    wmin = np.zeros((ng, N), dtype=np.float32)
    wmax = np.zeros((ng, N), dtype=np.float32)
    for g in range(ng):
        wmin[g] = np.min(W[g_idx == g], axis=0)
        wmax[g] = np.max(W[g_idx == g], axis=0)
    scales = ((wmax - wmin) / np.float32(3.0)).astype(np.float16)
    s32 = scales.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        z = np.where(s32 == 0, np.float32(0), np.rint(-wmin / s32))
    z = np.clip(z, 0, 3)
    zeros = z.astype(np.float16)
    u = np.clip(_quantise(W, s32[g_idx], -(1 << 20), 1 << 20) + z[g_idx].astype(np.int64), 0, 3)
    qweight = pack_q2(u)
    xr = np.random.default_rng(seed + M if x_seed is None else x_seed)
    X = xr.standard_normal((M, K)).astype(np.float16)
    return {"X": X, "qweight": qweight, "scales": scales, "zeros": zeros, "g_idx": g_idx,
            "u": u, "W": W, "M": M, "K": K, "N": N, "G": G}


def gen_w8a8(M: int, K: int, N: int, seed: int) -> dict:
    """W8A8 dynamic-quantisation inputs.

    Draw order: X ~ N(0,1) fp32 [M,K]; W ~ N(0, 0.02) fp32 indexed [K,N].
    The weight is quantised offline per output channel (column of W):
    ``Sw = fp32 colabsmax/127``, ``Wq = clip(rint(W/Sw), -127, 127)``, stored
    transposed as int8 ``[N, K]`` (K contiguous).  X stays fp32: it is
    quantised at run time by the path itself.
    """
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    W = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    Sw = _absmax_scale(W, axis=0, qmax=127.0)                      # [N]
    Wq = _quantise(W, Sw[None, :], -127, 127).astype(np.int8)
    Wq = np.ascontiguousarray(Wq.T)                                # [N, K]
    return {"X": X, "Wq": Wq, "Sw": Sw, "M": M, "K": K, "N": N}


def gen_w8a8_smooth(M: int, K: int, N: int, seed: int, n_outlier: int = 8,
                    outlier_scale: float = 20.0, alpha: float = 0.5) -> dict:
    """W8A8 inputs with outlier activation channels, and a SmoothQuant factor.

    Draw order: X ~ N(0,1) fp32 [M,K]; ``n_outlier`` distinct channels
    (``rng.choice``) of X multiplied by ``outlier_scale`` (activation outliers
    sit in a few fixed channels); W ~ N(0, 0.02) fp32 [K,N].  The factor is
    ``s[k] = max|X[:, k]|**alpha / max|W[k, :]|**(1 - alpha)`` in fp32
    (the usual migration-strength choice; alpha = 0.5).  The weight is folded
    and quantised offline: ``Ws = s[:, None] * W``, ``Sw = colabsmax(Ws)/127``,
    ``Wq = clip(rint(Ws/Sw), -127, 127)`` stored ``[N, K]``.  ``Wq0, Sw0`` are
    the same quantisation of W itself (no smoothing), for comparison.
    """
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    cols = rng.choice(K, size=n_outlier, replace=False)
    X[:, cols] *= np.float32(outlier_scale)
    W = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    ax = np.max(np.abs(X), axis=0).astype(np.float32)
    aw = np.max(np.abs(W), axis=1).astype(np.float32)
    smooth = (ax ** np.float32(alpha) / aw ** np.float32(1.0 - alpha)).astype(np.float32)
    Ws = (smooth[:, None] * W).astype(np.float32)
    Sw = _absmax_scale(Ws, axis=0, qmax=127.0)
    Wq = np.ascontiguousarray(_quantise(Ws, Sw[None, :], -127, 127).astype(np.int8).T)
    Sw0 = _absmax_scale(W, axis=0, qmax=127.0)
    Wq0 = np.ascontiguousarray(_quantise(W, Sw0[None, :], -127, 127).astype(np.int8).T)
    return {"X": X, "W": W, "smooth": smooth, "Wq": Wq, "Sw": Sw, "Wq0": Wq0, "Sw0": Sw0,
            "outlier_cols": cols, "M": M, "K": K, "N": N}


def gen_int8_mixed(M: int, K: int, N: int, seed: int, n_outlier: int = 8,
                   outlier_scale: float = 20.0) -> dict:
    """LLM.int8()-style inputs: fp16 activations with a few outlier channels, fp16 weight.

    Draw order: X ~ N(0,1) [M,K]; ``n_outlier`` distinct channels
    (``rng.choice``) multiplied by ``outlier_scale`` (most of their values
    then exceed 6); X rounded to fp16.  W ~ N(0, 0.02) fp32 [K,N], rounded to
    fp16 and stored ``[N, K]`` (K contiguous, one row per output channel).
    The weight stays in fp16: the decomposition quantises its regular part
    itself, after the split.
    """
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    cols = np.sort(rng.choice(K, size=n_outlier, replace=False))
    X[:, cols] *= np.float32(outlier_scale)
    X = X.astype(np.float16)
    W = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    W16 = np.ascontiguousarray(W.T.astype(np.float16))
    return {"X": X, "W16": W16, "outlier_cols": cols.astype(np.int32), "M": M, "K": K, "N": N}
