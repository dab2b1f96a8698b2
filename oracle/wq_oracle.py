"""Plain CPU oracle for the fused dequantize-and-multiply paths.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it and shares no code with it.

Everything here is the plain definition, written out step by step in numpy:
unpack the stored codes, dequantise them into a dense fp64 weight W, and
multiply with an fp64 matmul.  Nothing is blocked, fused or reordered.
The W8A8 path is the exception where the method fixes a precision: its
activation quantiser and its rescale epilogue are evaluated in fp32, with
the int32 accumulator computed exactly.

Sources (page title, then section):

* "GPTQ CUDA kernel walkthrough" (yelogs.com), section "CUDA核函數設計與實現":
  3-bit codes are taken from int32 words by shift-and-mask, and each weight
  is rebuilt as ``scale * q - zero`` with one scale and one zero per output
  column; the product is against a vector ``vec``.
* "Quantization CUDA" (tom-jerr.github.io):
  - "Dynamic Quantization": Y = X.W = (Sx*Xint).(Wint*Sw) = Sx*(Xint.Wint)*Sw,
    int8 multiply, int32 accumulation, float rescale;
  - "优化" (optimisation): the rescale is fused after the accumulation and
    the result is stored in bf16;
  - "Int8 Weight Only Quantization": Y = X.(Wint*Sw) with float multiply and
    fp32 accumulation;
  - "LLM.int8()": mixed-precision decomposition: columns of the activation
    matrix holding a value beyond a magnitude threshold (e.g. 6.0) and the
    matching weight rows are taken out and multiplied in 16-bit floating
    point; the rest is quantised to int8 (activations per token, weights per
    output channel) and multiplied in int8; the two results are added;
  - "Smoothquant": Y = (X diag(s)^-1) . (diag(s) W): the activations are
    divided by a per-input-channel factor s and the matching weight rows
    multiplied by it, before both are quantised to int8;
  - "量化粒度" (granularity): x = S*(q - Z); per-channel scales for weights,
    per-token for activations, group-wise (group 128) for int4;
  - "Weight Store" / "Int4 Weight Only Quantization": int4 codes are packed
    into a wider integer along the dimension one thread walks (K);
  - "Marlin 格式" (its part on working with the compute kernel): the
    asymmetric (AWQ) form rebuilds a weight as (W_int4 - Zero) * Scale from
    an unsigned 4-bit value, a zero and a scale of its group.
* "融合反量化与GEMM：LLM推理的CUDA内核优化实践" (zingnex.cn), "技术实现细节":
  symmetric int8 weights with one scale per group of 128 along K.
* "GPTQ算法解析" (intelliparadigm.com), section 4.1: group size 128,
  symmetric, act_order (a row -> group map that is not monotone in K).

Readings where the pages leave a step open (each one is also listed in the
design notes):

* The stored bit layouts are those the synthetic inputs define: 3-bit code
  ``i`` of a 32-row block at bit ``3i`` of the 96-bit little-endian value of
  three consecutive int32 words of one column; 4-bit row ``8r + j`` in
  nibble ``j`` of word ``r``, stored as ``q + 8``.
* 3-bit dequant uses the stored zero as given: ``w = scale*q - zero``.
* The asymmetric 4-bit form takes the unsigned nibble ``u`` (0..15) as the
  integer value and one fp16 zero and one fp16 scale per (group, column),
  both as given: ``w = (u - zero) * scale``.
* 2-bit codes, which "GPTQ CUDA kernel walkthrough" names only as a lower
  bit width still to support (its closing outlook): 16 per int32 along K,
  row ``16r + j`` in bits ``2j..2j+1`` of word ``r`` (the 4-bit order with
  2-bit fields), unsigned 0..3, rebuilt in the same asymmetric group-wise
  form ``w = (u - zero) * scale`` ("Quantization CUDA", "量化粒度":
  x = S*(q - Z) per group), since a symmetric 2-bit grid has no zero-centred
  form worth using.
* Outputs are overwritten (no accumulate into the caller's buffer), no bias.
* The activation quantiser divides (``absmax / 127`` then ``x / Sx``) in fp32
  with IEEE round-to-nearest, rounds half to even and clamps to [-127, 127];
  an all-zero row gets ``Sx = 0`` and all-zero codes.
* The epilogue is ``bf16_rne(f32(f32(Sx * f32(acc)) * Sw))``: two separately
  rounded fp32 multiplies, left to right, then round-to-nearest-even to bf16.
* LLM.int8(): X is fp16 and the weight is given in fp16, ``W16 [N, K]``; a
  column k is an outlier column when ``max_m |X[m, k]| > threshold``.  The
  16-bit side multiplies the fp16 outlier columns of X with the fp16 weight
  entries of the same k; the int8 side quantises the rest of X per row and
  the rest of W per output channel (the scales are taken over the regular
  columns only), multiplies exactly in int32 and rescales.  The output is
  the exact sum of the two parts (fp64); the GPU's fp16 output is compared
  with it at the floating-point tolerance, not bit for bit.
* SmoothQuant's ``X diag(s)^-1`` is one IEEE fp32 division per element,
  ``X[m, k] / s[k]``, before the per-row quantiser; ``diag(s) W`` is folded
  into the weight offline (fp32 multiply) before it is quantised.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bits_le", "unpack_q3", "unpack_u4", "unpack_q4", "dequant_q3", "dequant_q8_group",
    "materialize_q8_group",
    "dequant_q4_group", "dequant_q4_zp", "matvec_q3", "gemm_q8_group", "gemm_q4_group",
    "gemm_q4_zp", "unpack_u2", "gemm_q2_zp",
    "quantize_rows_int8", "w8a8_accumulate", "w8a8_epilogue",
    "bf16_rne_bits", "bf16_bits_to_f32", "gemm_w8a8", "smooth_activations",
    "smooth_weight", "gemm_w8a8_smooth", "int8_mixed_decompose",
]


# --------------------------------------------------------------------------
# Unpacking (the stored bit layouts)
# --------------------------------------------------------------------------

def bits_le(words: np.ndarray) -> np.ndarray:
    """Bits of int32 words, least significant first: ``[..., 32]`` of 0/1."""
    w = np.ascontiguousarray(words).astype("<u4")
    b = np.unpackbits(w.view(np.uint8).reshape(*w.shape, 4), axis=-1, bitorder="little")
    return b.reshape(*w.shape, 32)


def unpack_q3(qweight: np.ndarray) -> np.ndarray:
    """3-bit codes ``[K, N]`` (0..7) from int32 ``[3K/32, N]``.

    For column n and block b the three words 3b, 3b+1, 3b+2 are laid end to
    end, lowest word first, as one 96-bit string; code i of the block is bits
    3i, 3i+1, 3i+2 of that string (least significant first).
    """
    qweight = np.asarray(qweight)
    R, N = qweight.shape
    if R % 3:
        raise ValueError("3-bit weight must have a multiple of 3 word rows")
    nb = R // 3
    b = bits_le(qweight.reshape(nb, 3, N))             # [nb, 3, N, 32]
    b = b.transpose(0, 2, 1, 3).reshape(nb, N, 96)    # bit 32*j + t of word j
    trip = b.reshape(nb, N, 32, 3).astype(np.int64)   # bits 3i, 3i+1, 3i+2
    codes = trip[..., 0] + 2 * trip[..., 1] + 4 * trip[..., 2]   # [nb, N, 32]
    return codes.transpose(0, 2, 1).reshape(nb * 32, N)


def unpack_u4(qweight: np.ndarray) -> np.ndarray:
    """Unsigned 4-bit values ``[K, N]`` (0..15) from int32 ``[K/8, N]``.

    Row 8r + j is bits 4j..4j+3 of word r.
    """
    qweight = np.asarray(qweight)
    R, N = qweight.shape
    b = bits_le(qweight).astype(np.int64)             # [R, N, 32]
    nib = b.reshape(R, N, 8, 4)
    u = nib[..., 0] + 2 * nib[..., 1] + 4 * nib[..., 2] + 8 * nib[..., 3]  # [R, N, 8]
    return u.transpose(0, 2, 1).reshape(R * 8, N)


def unpack_q4(qweight: np.ndarray) -> np.ndarray:
    """Signed 4-bit codes ``[K, N]`` (-8..7): the unsigned value u minus 8."""
    return unpack_u4(qweight) - 8


def unpack_u2(qweight: np.ndarray) -> np.ndarray:
    """Unsigned 2-bit values ``[K, N]`` (0..3) from int32 ``[K/16, N]``.

    Row 16r + j is bits 2j, 2j+1 of word r.
    """
    qweight = np.asarray(qweight)
    R, N = qweight.shape
    b = bits_le(qweight).astype(np.int64)             # [R, N, 32]
    pair = b.reshape(R, N, 16, 2)
    u = pair[..., 0] + 2 * pair[..., 1]               # [R, N, 16]
    return u.transpose(0, 2, 1).reshape(R * 16, N)


# --------------------------------------------------------------------------
# Dequantisation to a dense fp64 weight
# --------------------------------------------------------------------------

def dequant_q3(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    """``W[k, n] = scale[n] * q[k, n] - zero[n]`` in fp64."""
    s = np.asarray(scales).astype(np.float64)[None, :]
    z = np.asarray(zeros).astype(np.float64)[None, :]
    return s * codes.astype(np.float64) - z


def dequant_q8_group(q: np.ndarray, scales: np.ndarray, G: int) -> np.ndarray:
    """``W[k, n] = scale[k // G, n] * q[k, n]`` in fp64."""
    K = q.shape[0]
    g = np.arange(K) // G
    return np.asarray(scales).astype(np.float64)[g, :] * q.astype(np.float64)


def materialize_q8_group(q: np.ndarray, scales: np.ndarray, G: int, out: str = "f32") -> np.ndarray:
    """The dense weight the separated (unfused) form writes before its GEMM.

    "融合反量化与GEMM：LLM推理的CUDA内核优化实践" (zingnex.cn), "CUDA内核架构":
    a standalone kernel dequantises the int8 weight to FP32 and writes all of
    it.  Here: the exact product ``scale * q`` (fp64: 24 + 8 bits, exact),
    rounded once to fp32; ``out="f16"`` rounds that fp32 weight once more to
    fp16 (both to nearest even), the fp16 weight a half-precision GEMM reads.
    """
    W32 = dequant_q8_group(q, scales, G).astype(np.float32)
    if out == "f32":
        return W32
    if out == "f16":
        return W32.astype(np.float16)
    raise ValueError(out)


def dequant_q4_group(q: np.ndarray, scales: np.ndarray, g_idx: np.ndarray | None,
                     G: int) -> np.ndarray:
    """``W[k, n] = scale[g_idx[k], n] * q[k, n]``; ``g_idx=None`` means ``k // G``."""
    K = q.shape[0]
    g = (np.arange(K) // G) if g_idx is None else np.asarray(g_idx).astype(np.int64)
    return np.asarray(scales).astype(np.float64)[g, :] * q.astype(np.float64)


def dequant_q4_zp(u: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                  g_idx: np.ndarray | None, G: int) -> np.ndarray:
    """``W[k, n] = (u[k, n] - zero[g, n]) * scale[g, n]``, ``g = g_idx[k]``
    (``k // G`` when ``g_idx`` is None), in fp64."""
    K = u.shape[0]
    g = (np.arange(K) // G) if g_idx is None else np.asarray(g_idx).astype(np.int64)
    z = np.asarray(zeros).astype(np.float64)[g, :]
    s = np.asarray(scales).astype(np.float64)[g, :]
    return (u.astype(np.float64) - z) * s


# --------------------------------------------------------------------------
# Weight-only products (fp64, unrounded)
# --------------------------------------------------------------------------

def matvec_q3(x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
              zeros: np.ndarray) -> np.ndarray:
    """``y = x . W`` with W the dequantised 3-bit weight; fp64, unrounded."""
    W = dequant_q3(unpack_q3(qweight), scales, zeros)
    return np.asarray(x).astype(np.float64) @ W


def gemm_q8_group(X: np.ndarray, q: np.ndarray, scales: np.ndarray, G: int) -> np.ndarray:
    """``Y = X . W`` with W the dequantised group-wise int8 weight; fp64."""
    W = dequant_q8_group(np.asarray(q), scales, G)
    return np.atleast_2d(np.asarray(X).astype(np.float64)) @ W


def gemm_q4_group(X: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                  g_idx: np.ndarray | None, G: int) -> np.ndarray:
    """``Y = X . W`` with W the dequantised group-wise 4-bit weight; fp64."""
    W = dequant_q4_group(unpack_q4(qweight), scales, g_idx, G)
    return np.atleast_2d(np.asarray(X).astype(np.float64)) @ W


def gemm_q4_zp(X: np.ndarray, qweight: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               g_idx: np.ndarray | None, G: int) -> np.ndarray:
    """``Y = X . W`` with W the dequantised asymmetric 4-bit weight; fp64."""
    W = dequant_q4_zp(unpack_u4(qweight), scales, zeros, g_idx, G)
    return np.atleast_2d(np.asarray(X).astype(np.float64)) @ W


def gemm_q2_zp(X: np.ndarray, qweight: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               g_idx: np.ndarray | None, G: int) -> np.ndarray:
    """``Y = X . W`` with W the dequantised asymmetric 2-bit weight; fp64.

    The same group-wise rebuild as the asymmetric 4-bit weight,
    ``(u - zero[g, n]) * scale[g, n]``, on the 2-bit values.
    """
    W = dequant_q4_zp(unpack_u2(qweight), scales, zeros, g_idx, G)
    return np.atleast_2d(np.asarray(X).astype(np.float64)) @ W


# --------------------------------------------------------------------------
# W8A8 dynamic quantisation
# --------------------------------------------------------------------------

def quantize_rows_int8(X: np.ndarray):
    """Per-row (per-token) symmetric int8 quantiser, evaluated in fp32.

    ``a = max|X[m, :]|``; ``Sx = a / 127``; ``Xq = clip(rint(X / Sx), -127, 127)``.
    A row with ``a == 0`` gets ``Sx = 0`` and all-zero codes.
    Returns ``(Xq int8 [M, K], Sx fp32 [M])``.
    """
    X = np.atleast_2d(np.asarray(X, dtype=np.float32))
    a = np.max(np.abs(X), axis=1)
    Sx = (a / np.float32(127.0)).astype(np.float32)
    Xq = np.zeros(X.shape, dtype=np.int8)
    for m in range(X.shape[0]):
        if a[m] == 0:
            continue
        r = np.rint(X[m] / Sx[m])                      # fp32 divide, round half even
        Xq[m] = np.clip(r, -127, 127).astype(np.int8)
    return Xq, Sx


def w8a8_accumulate(Xq: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """Exact int32 ``acc[m, n] = sum_k Xq[m, k] * Wq[n, k]``.

    Computed as an fp64 matmul: every partial sum is an integer of magnitude
    at most ``K * 127 * 127``, exact in fp64 while that stays below 2**53.
    """
    K = Xq.shape[1]
    if K * 127 * 127 >= 2 ** 53:
        raise ValueError("K too large for exact fp64 accumulation")
    acc = Xq.astype(np.float64) @ Wq.astype(np.float64).T
    acc_i = acc.astype(np.int64)
    if np.any(np.abs(acc_i) > 2 ** 31 - 1):
        raise OverflowError("accumulator exceeds int32")
    return acc_i.astype(np.int32)


def bf16_rne_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest-even; returns the uint16 bit patterns.

    Keeps the top 16 bits of the fp32 pattern, rounding on the 16 bits
    dropped: add 0x7FFF plus the lowest kept bit, then shift.  NaNs keep a
    quiet-NaN pattern.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    r = np.where(nan, ((u >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def w8a8_epilogue(acc: np.ndarray, Sx: np.ndarray, Sw: np.ndarray) -> np.ndarray:
    """``bf16_rne(f32(f32(Sx[m] * f32(acc[m, n])) * Sw[n]))`` as bf16 bits."""
    accf = acc.astype(np.float32)
    t = (np.asarray(Sx, np.float32)[:, None] * accf).astype(np.float32)
    y = (t * np.asarray(Sw, np.float32)[None, :]).astype(np.float32)
    return bf16_rne_bits(y)


def gemm_w8a8(X: np.ndarray, Wq: np.ndarray, Sw: np.ndarray) -> dict:
    """The whole W8A8 step: quantise X per row, int8 product, fused rescale.

    Returns ``Xq``, ``Sx``, the exact ``acc``, the bf16 output bits ``y_bits``
    and the unrounded fp64 ``y_exact = Sx * acc * Sw``.
    """
    Xq, Sx = quantize_rows_int8(X)
    acc = w8a8_accumulate(Xq, Wq)
    y_bits = w8a8_epilogue(acc, Sx, Sw)
    y_exact = (Sx.astype(np.float64)[:, None] * acc.astype(np.float64)
               * np.asarray(Sw, np.float64)[None, :])
    return {"Xq": Xq, "Sx": Sx, "acc": acc, "y_bits": y_bits, "y_exact": y_exact}


# --------------------------------------------------------------------------
# SmoothQuant folding around the W8A8 step
# --------------------------------------------------------------------------

def smooth_activations(X: np.ndarray, smooth: np.ndarray) -> np.ndarray:
    """``X . diag(s)^-1`` in fp32: ``X[m, k] / s[k]``, one IEEE division each."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float32))
    return (X / np.asarray(smooth, dtype=np.float32)[None, :]).astype(np.float32)


def smooth_weight(W: np.ndarray, smooth: np.ndarray) -> np.ndarray:
    """``diag(s) . W`` in fp32 for W indexed ``[K, N]`` (done once, offline)."""
    return (np.asarray(smooth, np.float32)[:, None] * np.asarray(W, np.float32)).astype(np.float32)


def gemm_w8a8_smooth(X: np.ndarray, smooth: np.ndarray, Wq: np.ndarray, Sw: np.ndarray) -> dict:
    """The W8A8 step on ``X . diag(s)^-1``; ``Wq, Sw`` quantise ``diag(s) . W``."""
    return gemm_w8a8(smooth_activations(X, smooth), Wq, Sw)


# --------------------------------------------------------------------------
# LLM.int8() mixed-precision decomposition
# --------------------------------------------------------------------------

def int8_mixed_decompose(X: np.ndarray, W16: np.ndarray, threshold: float) -> dict:
    """LLM.int8() mixed-precision decomposition of ``Y = X . W^T``.

    "Quantization CUDA" (tom-jerr.github.io), section "LLM.int8()", step by
    step, with ``X`` fp16 ``[M, K]`` and the fp16 weight ``W16`` ``[N, K]``
    (K contiguous; row n is output channel n):

    1. scan the activations: ``colmax[k] = max_m |X[m, k]|``; column k is an
       outlier column when ``colmax[k] > threshold``;
    2. split: the outlier part is those columns of X and the matching
       (k-indexed) weight entries ``W16[:, k]``; the regular part is the rest;
    3. int8 side: the regular part of X is quantised per token (row) and the
       regular part of W per output channel (row of ``W16``), both with the
       symmetric absmax/127 rule of ``quantize_rows_int8`` over the regular
       columns only; ``acc = Xq . Wq^T`` exactly in int32;
    4. 16-bit side: the outlier part stays in fp16 and is multiplied as is;
    5. the int8 result, dequantised (``Sx[m] * acc * Sw[n]``), plus the
       16-bit product is the output.

    Returns ``colmax`` (fp32), ``cols`` (ascending), ``Xq, Sx``, ``Wq, Sw``,
    ``acc``, the two parts in fp64 (``y_int8``, ``y_fp16``) and their exact
    sum ``y_exact``.
    """
    X = np.atleast_2d(np.asarray(X, dtype=np.float16)).astype(np.float32)
    W = np.atleast_2d(np.asarray(W16, dtype=np.float16)).astype(np.float32)
    if X.shape[1] != W.shape[1]:
        raise ValueError("X and W16 must share K")
    colmax = np.max(np.abs(X), axis=0).astype(np.float32)
    outlier = colmax > np.float32(threshold)
    cols = np.nonzero(outlier)[0]
    Xr = np.where(outlier[None, :], np.float32(0), X)
    Wr = np.where(outlier[None, :], np.float32(0), W)
    Xq, Sx = quantize_rows_int8(Xr)
    Wq, Sw = quantize_rows_int8(Wr)
    acc = w8a8_accumulate(Xq, Wq)
    y_int8 = Sx.astype(np.float64)[:, None] * acc.astype(np.float64) * Sw.astype(np.float64)[None, :]
    y_fp16 = X[:, cols].astype(np.float64) @ W[:, cols].astype(np.float64).T
    return {"colmax": colmax, "cols": cols.astype(np.int32), "Xq": Xq, "Sx": Sx, "Wq": Wq,
            "Sw": Sw, "acc": acc, "y_int8": y_int8, "y_fp16": y_fp16, "y_exact": y_int8 + y_fp16}
