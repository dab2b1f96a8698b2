"""Pins of the CPU oracle to facts fixed outside itself (CPU only).

Every test here checks the oracle (and the input packers it reads) against a
closed form, a hand-derived fixture under ``tests/golden``, an invariant, a
textbook/library routine or exact brute force, so that a dropped term, a
wrong sign, a wrong index or a transposed operand in the oracle fails one of
them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


# ---------------------------------------------------------------- layouts --

def test_q3_closed_form_words():
    for name, words, codes in read_golden("q3_pack_closed_forms.txt"):
        w = np.array([int(h, 16) for h in words.split()], dtype=np.uint32)
        c = np.array([int(v) for v in codes.split()])
        got = oracle.unpack_q3(w.view(np.int32).reshape(3, 1))[:, 0]
        assert np.array_equal(got, c), name
        packed = synth.pack_q3(c.reshape(32, 1)).view(np.uint32)[:, 0]
        assert np.array_equal(packed, w), name


def test_q4_closed_form_words():
    for name, word, codes in read_golden("q4_pack_closed_forms.txt"):
        w = np.array([int(word, 16)], dtype=np.uint32)
        q = np.array([int(v) for v in codes.split()])
        got = oracle.unpack_q4(w.view(np.int32).reshape(1, 1))[:, 0]
        assert np.array_equal(got, q), name
        packed = synth.pack_q4((q + 8).reshape(8, 1)).view(np.uint32)[0, 0]
        assert packed == w[0], name


def test_q3_roundtrip_multiblock():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 8, size=(96, 5))
    assert np.array_equal(oracle.unpack_q3(synth.pack_q3(codes)), codes)
    # Columns and blocks are independent: a code changed in one (block, column)
    # changes only that column's words of that block.
    c2 = codes.copy()
    c2[40, 3] ^= 5
    d = synth.pack_q3(c2) != synth.pack_q3(codes)
    assert set(zip(*np.nonzero(d))) <= {(3, 3), (4, 3), (5, 3)}


def test_q4_roundtrip_multirow():
    rng = np.random.default_rng(8)
    q = rng.integers(-8, 8, size=(64, 7))
    assert np.array_equal(oracle.unpack_q4(synth.pack_q4(q + 8)), q)


# ----------------------------------------------------------- 3-bit matvec --

def _q3_inputs(K, N, seed, codes=None, scales=None, zeros=None, x=None):
    rng = np.random.default_rng(seed)
    if codes is None:
        codes = rng.integers(0, 8, size=(K, N))
    if scales is None:
        scales = rng.uniform(0.005, 0.02, N).astype(np.float32)
    if zeros is None:
        zeros = (scales * rng.integers(0, 8, N)).astype(np.float32)
    if x is None:
        x = rng.standard_normal(K).astype(np.float32)
    return x, synth.pack_q3(codes), scales, zeros, codes


def test_q3_all_zero_codes_closed_form():
    # w = scale*0 - zero, so y[n] = -zero[n] * sum(x).
    x, qw, s, z, _ = _q3_inputs(64, 12, 1, codes=np.zeros((64, 12), dtype=np.int64))
    y = oracle.matvec_q3(x, qw, s, z)
    expect = -z.astype(np.float64) * np.sum(x.astype(np.float64))
    assert np.allclose(y, expect, rtol=1e-13, atol=1e-15)


def test_q3_one_hot_rows():
    # x = e_k selects row k of W: y[n] = scale[n]*q[k, n] - zero[n] for every k.
    K, N = 64, 9
    _, qw, s, z, codes = _q3_inputs(K, N, 2)
    for k in range(K):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = oracle.matvec_q3(x, qw, s, z)
        expect = s.astype(np.float64) * codes[k] - z.astype(np.float64)
        assert np.array_equal(y, expect), k


def test_q3_integer_case_brute_force():
    # scale 1, integer zero and small integer x: y is an exact integer.
    K, N = 64, 6
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 8, size=(K, N))
    z = rng.integers(0, 8, size=N)
    x = rng.integers(-4, 5, size=K)
    y = oracle.matvec_q3(x.astype(np.float32), synth.pack_q3(codes),
                         np.ones(N, np.float32), z.astype(np.float32))
    for n in range(N):
        acc = 0
        for k in range(K):
            acc += int(x[k]) * (int(codes[k, n]) - int(z[n]))
        assert y[n] == acc


def _gamma(n, u=Fraction(1, 2 ** 53)):
    """Higham's gamma_n = n u / (1 - n u) (u the unit roundoff, fp64 by default)."""
    return n * u / (1 - n * u)


def test_q3_against_exact_rationals():
    # 32x8 tile: fp64 oracle vs exact Fraction arithmetic on the stored fp32
    # values, within the forward error bound of an fp64 dot product: each
    # weight scale*q - zero is at most one rounding (scale*q is exact), each
    # product one more, the sum of K terms K - 1 more, so
    # |y - exact| <= gamma_{K+2} * sum_k |x_k| |w_k|.
    K, N = 32, 8
    x, qw, s, z, codes = _q3_inputs(K, N, 4)
    y = oracle.matvec_q3(x, qw, s, z)
    for n in range(N):
        terms = [Fraction(float(x[k])) * (Fraction(float(s[n])) * int(codes[k, n]) - Fraction(float(z[n])))
                 for k in range(K)]
        exact = sum(terms)
        assert abs(Fraction(float(y[n])) - exact) <= _gamma(K + 2) * sum(abs(t) for t in terms)


def test_q8_and_q4_forward_error_bound():
    # Group-wise int8 and act-order 4-bit tiles against exact rationals, with
    # the same rigorous fp64 dot-product bound (scale*q is exact in fp64, so
    # only the products and the K - 1 additions round).
    K, N, G = 256, 6, 64
    d8 = synth.gen_q8_group(1, K, N, G, seed=31)
    y8 = oracle.gemm_q8_group(d8["X"], d8["q"], d8["scales"], G)
    d4 = synth.gen_q4_group(1, K, N, 32, seed=32)
    y4 = oracle.gemm_q4_group(d4["X"], d4["qweight"], d4["scales"], d4["g_idx"], 32)
    u4 = oracle.unpack_u4(d4["qweight"])
    for n in range(N):
        t8 = [Fraction(float(d8["X"][0, k])) * Fraction(float(d8["scales"][k // G, n])) * int(d8["q"][k, n])
              for k in range(K)]
        t4 = [Fraction(float(d4["X"][0, k])) * Fraction(float(d4["scales"][d4["g_idx"][k], n]))
              * (int(u4[k, n]) - 8) for k in range(K)]
        for y, t in ((y8, t8), (y4, t4)):
            assert abs(Fraction(float(y[0, n])) - sum(t)) <= _gamma(K + 1) * sum(abs(v) for v in t)


def test_q3_scaling_invariance():
    # y is linear in x and in (scale, zero) jointly.
    x, qw, s, z, _ = _q3_inputs(96, 10, 5)
    y = oracle.matvec_q3(x, qw, s, z)
    assert np.array_equal(oracle.matvec_q3(2 * x, qw, s, z), 2 * y)
    assert np.allclose(oracle.matvec_q3(x, qw, 4 * s, 4 * z), 4 * y, rtol=1e-14, atol=0)


# --------------------------------------------------------- int8 group-wise --

def test_q8_group_one_hot_uses_group_of_row():
    K, N, G = 256, 5, 64
    d = synth.gen_q8_group(1, K, N, G, seed=11)
    for k in (0, 63, 64, 127, 128, 255):
        x = np.zeros(K, np.float16)
        x[k] = 1
        y = oracle.gemm_q8_group(x, d["q"], d["scales"], G)[0]
        expect = d["scales"][k // G].astype(np.float64) * d["q"][k].astype(np.float64)
        assert np.array_equal(y, expect), k


def test_q8_group_power_of_two_scales_closed_form():
    # scale[g, n] = 2**g and x = 1: y[n] = sum_g 2**g * (sum of codes of group g).
    K, N, G = 512, 7, 128
    rng = np.random.default_rng(12)
    q = rng.integers(-127, 128, size=(K, N)).astype(np.int8)
    scales = np.array([[2.0 ** g] * N for g in range(K // G)], dtype=np.float32)
    y = oracle.gemm_q8_group(np.ones(K, np.float16), q, scales, G)[0]
    for n in range(N):
        expect = 0
        for g in range(K // G):
            expect += 2 ** g * int(q[g * G:(g + 1) * G, n].astype(np.int64).sum())
        assert y[n] == expect


def test_q8_equal_scales_reduce_to_integer_dot():
    # One scale everywhere: y = s * (x . q), with x small integers -> integer dot product.
    K, N, G = 256, 16, 128
    rng = np.random.default_rng(13)
    q = rng.integers(-127, 128, size=(K, N)).astype(np.int8)
    x = rng.integers(-3, 4, size=(2, K))
    s = np.float32(0.25)
    y = oracle.gemm_q8_group(x.astype(np.float16), q, np.full((K // G, N), s), G)
    assert np.array_equal(y, float(s) * np.dot(x.astype(np.int64), q.astype(np.int64)))


def test_q8_zero_codes():
    d = synth.gen_q8_group(3, 256, 8, 128, seed=14)
    y = oracle.gemm_q8_group(d["X"], np.zeros_like(d["q"]), d["scales"], 128)
    assert np.all(y == 0)


# ---------------------------------------------------------- 4-bit grouped --

def test_q4_gidx_default_equals_k_over_g():
    d = synth.gen_q4_group(2, 256, 12, 64, seed=21, act_order=False)
    a = oracle.gemm_q4_group(d["X"], d["qweight"], d["scales"], None, 64)
    b = oracle.gemm_q4_group(d["X"], d["qweight"], d["scales"], d["g_idx"], 64)
    assert np.array_equal(a, b)


def test_q4_one_hot_act_order():
    K, N, G = 256, 9, 64
    d = synth.gen_q4_group(1, K, N, G, seed=22, act_order=True)
    assert not np.all(np.diff(d["g_idx"]) >= 0)       # really out of order
    for k in (0, 1, 7, 8, 100, 255):
        x = np.zeros(K, np.float16)
        x[k] = 1
        y = oracle.gemm_q4_group(x, d["qweight"], d["scales"], d["g_idx"], G)[0]
        expect = d["scales"][d["g_idx"][k]].astype(np.float64) * d["codes"][k]
        assert np.array_equal(y, expect), k


def test_q4_consistent_k_permutation_invariance():
    # Reordering K in codes, x and g_idx together leaves y unchanged (exact
    # here: power-of-two scales and small integer activations).
    K, N, G = 128, 6, 32
    rng = np.random.default_rng(23)
    q = rng.integers(-8, 8, size=(K, N))
    g_idx = rng.permutation(np.repeat(np.arange(K // G), G)).astype(np.int32)
    scales = (2.0 ** rng.integers(-3, 3, size=(K // G, N))).astype(np.float16)
    x = rng.integers(-3, 4, size=(1, K)).astype(np.float16)
    y = oracle.gemm_q4_group(x, synth.pack_q4(q + 8), scales, g_idx, G)
    p = rng.permutation(K)
    y2 = oracle.gemm_q4_group(x[:, p], synth.pack_q4(q[p] + 8), scales, g_idx[p], G)
    assert np.array_equal(y, y2)


def test_q4_zero_codes():
    K, N, G = 64, 4, 32
    qw = synth.pack_q4(np.full((K, N), 8))
    y = oracle.gemm_q4_group(np.ones((3, K), np.float16), qw,
                             np.ones((K // G, N), np.float16), None, G)
    assert np.all(y == 0)


def test_q4_generator_groups_balanced():
    d = synth.gen_q4_group(1, 4096, 16, 128, seed=1300)
    counts = np.bincount(d["g_idx"], minlength=32)
    assert np.all(counts == 128)
    assert d["codes"].min() >= -8 and d["codes"].max() <= 7


# ------------------------------------------------------------------- W8A8 --

def test_w8a8_quantiser_ties_and_extremes():
    # Row absmax 127 -> Sx = 1 exactly; halves round to even.
    X = np.array([[127.0, 2.5, -2.5, 3.5, -3.5, 0.5, 1.5, -127.0]], np.float32)
    Xq, Sx = oracle.quantize_rows_int8(X)
    assert Sx[0] == np.float32(1.0)
    assert Xq[0].tolist() == [127, 2, -2, 4, -4, 0, 2, -127]


def test_w8a8_quantiser_zero_row_and_bound():
    rng = np.random.default_rng(31)
    X = rng.standard_normal((4, 512)).astype(np.float32)
    X[2] = 0
    Xq, Sx = oracle.quantize_rows_int8(X)
    assert Sx[2] == 0 and np.all(Xq[2] == 0)
    for m in (0, 1, 3):
        amax = np.max(np.abs(X[m]))
        assert Sx[m] == np.float32(amax) / np.float32(127)
        assert np.abs(Xq[m]).max() == 127
        assert Xq[m][np.argmax(np.abs(X[m]))] == np.sign(X[m][np.argmax(np.abs(X[m]))]) * 127
        err = np.abs(X[m].astype(np.float64) - Sx[m].astype(np.float64) * Xq[m])
        assert np.all(err <= 0.5 * Sx[m] * (1 + 1e-6))


def test_w8a8_rearrangement_identity():
    # Y = (Sx*Xint).(Wint*Sw) = Sx*(Xint.Wint)*Sw ("Quantization CUDA", Dynamic Quantization).
    d = synth.gen_w8a8(8, 256, 24, seed=32)
    r = oracle.gemm_w8a8(d["X"], d["Wq"], d["Sw"])
    lhs = ((r["Sx"].astype(np.float64)[:, None] * r["Xq"])
           @ (d["Wq"].T.astype(np.float64) * d["Sw"].astype(np.float64)[None, :]))
    assert np.allclose(lhs, r["y_exact"], rtol=1e-12, atol=1e-300)
    # and the quantised product approximates the float one
    ref = d["X"].astype(np.float64) @ (d["Wq"].T.astype(np.float64) * d["Sw"][None, :])
    assert np.linalg.norm(r["y_exact"] - ref) / np.linalg.norm(ref) < 0.02


def test_w8a8_accumulator_exact_vs_int64():
    rng = np.random.default_rng(33)
    Xq = rng.integers(-127, 128, size=(64, 8192)).astype(np.int8)
    Wq = rng.integers(-127, 128, size=(64, 8192)).astype(np.int8)
    acc = oracle.w8a8_accumulate(Xq, Wq)
    ref = Xq.astype(np.int64) @ Wq.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), ref)
    # extreme magnitudes: all +127 -> K * 127^2 exactly
    big = oracle.w8a8_accumulate(np.full((1, 8192), 127, np.int8), np.full((1, 8192), -127, np.int8))
    assert big[0, 0] == -8192 * 127 * 127


def test_bf16_and_fp16_ties_golden():
    for fmt, inp, exp in read_golden("rounding_ties.txt"):
        v = np.array([float(inp)], np.float32)
        if fmt == "bf16":
            got = oracle.bf16_bits_to_f32(oracle.bf16_rne_bits(v))[0]
        else:
            got = v.astype(np.float16)[0]
        assert float(got) == float(exp), (fmt, inp)


def test_bf16_matches_torch_cpu():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(34)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1e-40, -1e-40, 3.0e38, -3.0e38]]).astype(np.float32)
    ours = oracle.bf16_rne_bits(v)
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_w8a8_epilogue_ties_through_path():
    # Sx = Sw = 1: the epilogue is bf16(acc); 257 -> 256, 259 -> 260, 514 -> 512, 518 -> 520.
    acc = np.array([[257, 259, 514, 518, -257]], np.int32)
    y = oracle.bf16_bits_to_f32(oracle.w8a8_epilogue(acc, np.ones(1, np.float32), np.ones(5, np.float32)))
    assert y.tolist() == [[256.0, 260.0, 512.0, 520.0, -256.0]]


def test_w8a8_epilogue_per_row_and_per_column_scales():
    # tests/golden/w8a8_epilogue_worked.txt: distinct per-row Sx and
    # per-column Sw, M != N and M == N, and two bf16 roundings, by hand.
    for name, M, N, acc, sx, sw, y in read_golden("w8a8_epilogue_worked.txt"):
        M, N = int(M), int(N)
        acc = np.array([int(v) for v in acc.split()], np.int32).reshape(M, N)
        sx = np.array([float(v) for v in sx.split()], np.float32)
        sw = np.array([float(v) for v in sw.split()], np.float32)
        got = oracle.bf16_bits_to_f32(oracle.w8a8_epilogue(acc, sx, sw))
        assert got.ravel().tolist() == [float(v) for v in y.split()], name


# ------------------------------------------------- asymmetric 4-bit (AWQ) --

def test_q4_zp_worked_examples():
    for name, words, G, zeros, scales, x, y in read_golden("q4_zp_worked.txt"):
        w = np.array([int(h, 16) for h in words.split()], dtype=np.uint32)
        qw = w.view(np.int32).reshape(-1, 1)
        z = np.array([float(v) for v in zeros.split()]).reshape(-1, 1)
        s = np.array([float(v) for v in scales.split()]).reshape(-1, 1)
        xv = np.array([float(v) for v in x.split()]).reshape(1, -1)
        got = oracle.gemm_q4_zp(xv, qw, s, z, None, int(G))
        assert got.shape == (1, 1)
        assert got[0, 0] == float(y), name


def test_q4_zp_unsigned_nibbles_closed_form():
    # nibble j of 0x76543210 is j; of 0xFEDCBA98 it is 8 + j.
    w = np.array([0x76543210, 0xFEDCBA98], dtype=np.uint32).view(np.int32).reshape(2, 1)
    assert np.array_equal(oracle.unpack_u4(w)[:, 0], np.arange(16))
    assert np.array_equal(oracle.unpack_q4(w)[:, 0], np.arange(16) - 8)


def test_q4_zp_zero_eight_is_the_symmetric_form():
    # With every zero 8 the asymmetric form is the symmetric one (u = q + 8).
    d = synth.gen_q4_group(3, 512, 40, 128, seed=61, act_order=True)
    z = np.full_like(d["scales"], 8.0)
    a = oracle.gemm_q4_zp(d["X"], d["qweight"], d["scales"], z, d["g_idx"], 128)
    b = oracle.gemm_q4_group(d["X"], d["qweight"], d["scales"], d["g_idx"], 128)
    assert np.array_equal(a, b)


def test_q4_zp_shift_invariance():
    # Adding the same constant to every value and zero of a group leaves W.
    rng = np.random.default_rng(62)
    K, N, G = 128, 8, 32
    u = rng.integers(0, 14, size=(K, N))
    z = rng.integers(0, 14, size=(K // G, N)).astype(np.float64)
    s = rng.uniform(0.01, 0.1, size=(K // G, N))
    x = rng.standard_normal((2, K))
    a = oracle.gemm_q4_zp(x, synth.pack_q4(u), s, z, None, G)
    b = oracle.gemm_q4_zp(x, synth.pack_q4(u + 1), s, z + 1, None, G)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_q4_zp_group_index_and_column_brute_force():
    # Tiny case summed term by term with exact rationals (scales and zeros
    # picked as dyadic values), against the fp64 oracle.
    rng = np.random.default_rng(63)
    K, N, G = 16, 3, 8
    u = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(K // G, N)) / 2.0
    s = rng.integers(1, 9, size=(K // G, N)) / 8.0
    x = rng.integers(-3, 4, size=(1, K)).astype(np.float64)
    got = oracle.gemm_q4_zp(x, synth.pack_q4(u), s, z, None, G)[0]
    for n in range(N):
        acc = Fraction(0)
        for k in range(K):
            g = k // G
            acc += Fraction(x[0, k]) * (Fraction(int(u[k, n])) - Fraction(z[g, n])) * Fraction(s[g, n])
        assert got[n] == float(acc), n


def test_q4_zp_generator_roundtrip_bound():
    d = synth.gen_q4_zp(1, 512, 64, 64, seed=64)
    W = oracle.dequant_q4_zp(oracle.unpack_u4(d["qweight"]), d["scales"], d["zeros"], None, 64)
    s = d["scales"].astype(np.float64)[np.arange(512) // 64]
    assert np.all(np.abs(W - d["W"]) <= s * (0.5 + 1e-3) + 1e-12)


# ------------------------------------------------------ asymmetric 2-bit --

def test_q2_zp_worked_examples():
    for name, words, G, zeros, scales, x, y in read_golden("q2_zp_worked.txt"):
        w = np.array([int(h, 16) for h in words.split()], dtype=np.uint32)
        qw = w.view(np.int32).reshape(-1, 1)
        z = np.array([float(v) for v in zeros.split()]).reshape(-1, 1)
        s = np.array([float(v) for v in scales.split()]).reshape(-1, 1)
        xv = np.array([float(v) for v in x.split()]).reshape(1, -1)
        got = oracle.gemm_q2_zp(xv, qw, s, z, None, int(G))
        assert got.shape == (1, 1)
        assert got[0, 0] == float(y), name


def test_q2_closed_form_words():
    w = np.array([0xE4E4E4E4, 0x1B1B1B1B, 0xC0000000, 0x00000001], dtype=np.uint32)
    u = oracle.unpack_u2(w.view(np.int32).reshape(4, 1))[:, 0]
    assert np.array_equal(u[0:16], np.arange(16) % 4)
    assert np.array_equal(u[16:32], 3 - np.arange(16) % 4)
    assert np.array_equal(u[32:48], np.r_[np.zeros(15, int), 3])
    assert np.array_equal(u[48:64], np.r_[1, np.zeros(15, int)])


def test_q2_roundtrip_and_generator_bound():
    rng = np.random.default_rng(65)
    u = rng.integers(0, 4, size=(96, 7))
    assert np.array_equal(oracle.unpack_u2(synth.pack_q2(u)), u)
    d = synth.gen_q2_zp(1, 512, 48, 128, seed=66, act_order=True)
    assert np.array_equal(oracle.unpack_u2(d["qweight"]), d["u"])
    W = oracle.dequant_q4_zp(d["u"], d["scales"], d["zeros"], d["g_idx"], 128)
    s = d["scales"].astype(np.float64)[d["g_idx"]]
    assert np.all(np.abs(W - d["W"]) <= s * (0.5 + 1e-3) + 1e-12)


def test_q2_matches_the_same_values_as_4bit():
    # The same unsigned values packed as 2-bit and as 4-bit fields go through
    # two independent unpackers into the same asymmetric rebuild.
    d = synth.gen_q2_zp(3, 256, 24, 64, seed=67, act_order=True)
    a = oracle.gemm_q2_zp(d["X"], d["qweight"], d["scales"], d["zeros"], d["g_idx"], 64)
    b = oracle.gemm_q4_zp(d["X"], synth.pack_q4(d["u"]), d["scales"], d["zeros"], d["g_idx"], 64)
    assert np.array_equal(a, b)


def test_q2_group_brute_force():
    rng = np.random.default_rng(68)
    K, N, G = 32, 3, 16
    u = rng.integers(0, 4, size=(K, N))
    z = rng.integers(0, 7, size=(K // G, N)) / 2.0
    s = rng.integers(1, 9, size=(K // G, N)) / 8.0
    x = rng.integers(-3, 4, size=(1, K)).astype(np.float64)
    got = oracle.gemm_q2_zp(x, synth.pack_q2(u), s, z, None, G)[0]
    for n in range(N):
        acc = Fraction(0)
        for k in range(K):
            g = k // G
            acc += Fraction(x[0, k]) * (Fraction(int(u[k, n])) - Fraction(z[g, n])) * Fraction(s[g, n])
        assert got[n] == float(acc), n


# ------------------------------------------------------------ SmoothQuant --

def test_smooth_ones_is_plain_w8a8():
    d = synth.gen_w8a8(5, 256, 32, seed=71)
    a = oracle.gemm_w8a8_smooth(d["X"], np.ones(256, np.float32), d["Wq"], d["Sw"])
    b = oracle.gemm_w8a8(d["X"], d["Wq"], d["Sw"])
    for key in ("Xq", "Sx", "acc", "y_bits"):
        assert np.array_equal(a[key], b[key]), key


def test_smooth_identity_exact_case():
    # (X diag(s)^-1)(diag(s) W) = X W.  Built so that every step is exact:
    # s = powers of two, X / s integers with row max 127 (Sx = 1), s W
    # integers with column max 127 (Sw = 1); the result must be X . W.
    rng = np.random.default_rng(72)
    M, K, N = 4, 64, 16
    s = (2.0 ** rng.integers(-3, 4, size=K)).astype(np.float32)
    Xs = rng.integers(-127, 128, size=(M, K))
    Xs[:, 0] = 127
    Ws = rng.integers(-127, 128, size=(K, N))
    Ws[1, :] = -127
    X = (Xs * s[None, :]).astype(np.float32)
    W = (Ws / s[:, None]).astype(np.float32)
    folded = oracle.smooth_weight(W, s)
    assert np.array_equal(folded, Ws.astype(np.float32))
    Wq = np.ascontiguousarray(Ws.T.astype(np.int8))
    r = oracle.gemm_w8a8_smooth(X, s, Wq, np.ones(N, np.float32))
    assert np.array_equal(r["Sx"], np.ones(M, np.float32))
    assert np.array_equal(r["Xq"], Xs.astype(np.int8))
    assert np.array_equal(r["y_exact"], X.astype(np.float64) @ W.astype(np.float64))


def test_smooth_reduces_error_with_outlier_channels():
    # Few activation channels 20x larger: per-token int8 quantisation of X
    # crushes the other channels; dividing them out (and folding s into W)
    # brings the product much closer to X . W.
    d = synth.gen_w8a8_smooth(32, 1024, 64, seed=synth.SEEDS["w8a8_smooth"])
    ref = d["X"].astype(np.float64) @ d["W"].astype(np.float64)
    plain = oracle.gemm_w8a8(d["X"], d["Wq0"], d["Sw0"])["y_exact"]
    smooth = oracle.gemm_w8a8_smooth(d["X"], d["smooth"], d["Wq"], d["Sw"])["y_exact"]
    e_plain = np.linalg.norm(plain - ref) / np.linalg.norm(ref)
    e_smooth = np.linalg.norm(smooth - ref) / np.linalg.norm(ref)
    assert e_smooth < 0.5 * e_plain, (e_plain, e_smooth)


# -------------------------------------------------------------- LLM.int8() --

def _mixed_fixture():
    rows = {k: v for k, v in read_golden("int8_mixed_worked.txt")}
    f = lambda key: np.array([float(t) for t in rows[key].split()])
    return rows, f


def test_mixed_worked_example():
    # tests/golden/int8_mixed_worked.txt: every intermediate of the page's
    # steps, derived by hand; the outlier weight entries (5 and -1.5) enter
    # in fp16, and the per-channel scales cover the regular columns only.
    rows, f = _mixed_fixture()
    X = f("X").reshape(2, 4).astype(np.float16)
    W = f("W").reshape(2, 4).astype(np.float16)
    r = oracle.int8_mixed_decompose(X, W, threshold=float(rows["thresh"]))
    assert r["colmax"].tolist() == f("colmax").tolist()
    assert r["cols"].tolist() == [int(v) for v in rows["cols"].split()]
    assert r["Xq"].ravel().tolist() == f("Xq").astype(int).tolist()
    assert r["Sx"].tolist() == f("Sx").tolist()
    assert r["Wq"].ravel().tolist() == f("Wq").astype(int).tolist()
    assert r["Sw"].tolist() == f("Sw").tolist()
    assert r["acc"].ravel().tolist() == f("acc").astype(int).tolist()
    assert r["y_exact"].ravel().tolist() == f("y").tolist()


def test_mixed_outlier_rows_stay_fp16():
    # Changing only the outlier weight entries changes y by exactly
    # X[:, cols] . dW (the 16-bit side), and leaves the int8 side alone, even
    # when the new entries are far off the regular part's int8 grid.
    rows, f = _mixed_fixture()
    X = f("X").reshape(2, 4).astype(np.float16)
    W = f("W").reshape(2, 4).astype(np.float16)
    W2 = W.copy()
    W2[:, 2] = np.array([1000.0, -0.0009765625], np.float16)
    a = oracle.int8_mixed_decompose(X, W, 6.0)
    b = oracle.int8_mixed_decompose(X, W2, 6.0)
    for key in ("Wq", "Sw", "Xq", "Sx", "acc"):
        assert np.array_equal(a[key], b[key]), key
    d = X[:, 2:3].astype(np.float64) @ (W2[:, 2:3].astype(np.float64) - W[:, 2:3].astype(np.float64)).T
    assert np.array_equal(b["y_exact"] - a["y_exact"], d)


def test_mixed_no_outliers_is_plain_w8a8():
    # Above every value: no column is taken out; the int8 side is W8A8 with
    # the weight quantised per output channel over all of K.
    rng = np.random.default_rng(81)
    X16 = rng.standard_normal((6, 256)).astype(np.float16)
    W16 = rng.normal(0, 0.02, size=(32, 256)).astype(np.float16)
    r = oracle.int8_mixed_decompose(X16, W16, threshold=1e30)
    Wq, Sw = oracle.quantize_rows_int8(W16.astype(np.float32))
    p = oracle.gemm_w8a8(X16.astype(np.float32), Wq, Sw)
    assert r["cols"].size == 0 and np.all(r["y_fp16"] == 0)
    for key in ("Xq", "Sx", "acc"):
        assert np.array_equal(r[key], p[key]), key
    assert np.array_equal(r["Wq"], Wq) and np.array_equal(r["Sw"], Sw)
    assert np.array_equal(r["y_exact"], p["y_exact"])


def test_mixed_all_outliers_is_the_fp16_product():
    # Below every magnitude: every column is 16-bit, the int8 side is empty
    # and y is X . W^T of the fp16 values, exactly.
    rng = np.random.default_rng(82)
    M, K, N = 3, 64, 16
    X = rng.standard_normal((M, K)).astype(np.float16)
    X[:, 0] = 1                                       # no all-zero column
    W = rng.normal(0, 0.02, size=(N, K)).astype(np.float16)
    r = oracle.int8_mixed_decompose(X, W, threshold=-1.0)
    assert r["cols"].size == K
    assert np.all(r["Xq"] == 0) and np.all(r["Sx"] == 0) and np.all(r["Wq"] == 0) and np.all(r["Sw"] == 0)
    exact = [[sum(Fraction(float(X[m, k])) * Fraction(float(W[n, k])) for k in range(K))
              for n in range(N)] for m in range(M)]
    # every product of two fp16 values is exact in fp64; the sum of 64 such
    # terms is within gamma_64 * sum |x w| of the exact rational
    u = Fraction(1, 2 ** 53)
    g = 64 * u / (1 - 64 * u)
    for m in range(M):
        for n in range(N):
            bound = g * sum(abs(Fraction(float(X[m, k])) * Fraction(float(W[n, k]))) for k in range(K))
            assert abs(Fraction(float(r["y_exact"][m, n])) - exact[m][n]) <= bound


def test_mixed_reduces_error_with_outlier_channels():
    d = synth.gen_int8_mixed(32, 1024, 64, seed=synth.SEEDS["int8_mixed"])
    ref = d["X"].astype(np.float64) @ d["W16"].astype(np.float64).T
    Wq, Sw = oracle.quantize_rows_int8(d["W16"].astype(np.float32))
    plain = oracle.gemm_w8a8(d["X"].astype(np.float32), Wq, Sw)["y_exact"]
    mixed = oracle.int8_mixed_decompose(d["X"], d["W16"], 6.0)
    assert np.array_equal(mixed["cols"], d["outlier_cols"])
    e_plain = np.linalg.norm(plain - ref) / np.linalg.norm(ref)
    e_mixed = np.linalg.norm(mixed["y_exact"] - ref) / np.linalg.norm(ref)
    assert e_mixed < 0.5 * e_plain, (e_plain, e_mixed)


# ---------------------------------------------- separated form's weight --

def test_materialize_q8_worked_example():
    # tests/golden/q8_materialize_worked.txt: a product that rounds to an fp16
    # tie only after the fp32 rounding (two-step rounding pinned by hand).
    for name, sc, q, b32, b16 in read_golden("q8_materialize_worked.txt"):
        scale = np.array([[np.float32(int(sc) * 2.0 ** -26)]], np.float32)
        assert float(scale[0, 0]) == int(sc) * 2.0 ** -26   # the scale is an fp32 number
        qq = np.array([[int(q)]], np.int8)
        w32 = oracle.materialize_q8_group(qq, scale, 1, "f32")
        w16 = oracle.materialize_q8_group(qq, scale, 1, "f16")
        assert w32.dtype == np.float32 and w16.dtype == np.float16
        assert int(w32.view(np.uint32)[0, 0]) == int(b32, 16), name
        assert int(w16.view(np.uint16)[0, 0]) == int(b16, 16), name


def test_materialize_q8_exact_with_power_of_two_scales_and_groups():
    # Power-of-two scales: every product is exact in fp32 (and in fp16 for
    # |q| <= 127 at these exponents), and row k takes the scale of group
    # k // G: rows 0..31 of group 0 (scale 2^-7), rows 32..63 of group 1
    # (scale 2^-3).
    rng = np.random.default_rng(5)
    K, N, G = 64, 16, 32
    q = rng.integers(-127, 128, size=(K, N)).astype(np.int8)
    s = np.empty((2, N), np.float32)
    s[0], s[1] = 2.0 ** -7, 2.0 ** -3
    w32 = oracle.materialize_q8_group(q, s, G, "f32").astype(np.float64)
    w16 = oracle.materialize_q8_group(q, s, G, "f16").astype(np.float64)
    exact = np.vstack([q[:32].astype(np.float64) / 128.0, q[32:].astype(np.float64) / 8.0])
    assert np.array_equal(w32, exact)
    assert np.array_equal(w16, exact)


def test_materialize_q8_within_one_rounding_of_exact():
    # Arbitrary fp32 scales: the fp32 weight is within half an fp32 ulp of
    # the exact product, the fp16 weight within half an fp16 ulp plus half an
    # fp32 ulp; a naive product with the fp32 weight stays within the
    # weight's relative error of the exact GEMM.
    d = synth.gen_q8_group(3, 256, 64, 128, seed=17)
    q, s = d["q"], d["scales"]
    ex = q.astype(np.float64) * np.repeat(s.astype(np.float64), 128, axis=0)
    w32 = oracle.materialize_q8_group(q, s, 128, "f32").astype(np.float64)
    w16 = oracle.materialize_q8_group(q, s, 128, "f16").astype(np.float64)
    assert np.all(np.abs(w32 - ex) <= 2.0 ** -24 * np.abs(ex))
    assert np.all(np.abs(w16 - ex) <= (2.0 ** -11 + 2.0 ** -24) * np.abs(ex) + 2.0 ** -25)
    X = d["X"].astype(np.float64)
    y = X @ w32
    y_ex = oracle.gemm_q8_group(d["X"], q, s, 128)
    assert np.all(np.abs(y - y_ex) <= 2.0 ** -24 * (np.abs(X) @ np.abs(ex)) * 1.0001)
