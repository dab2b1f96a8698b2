"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Bars: integer results (unpacked codes, the W8A8 activation codes, scales and
int32 accumulators, and the bf16 output bits of the fixed-order epilogue)
are compared bit for bit.  Floating outputs of the weight-only paths must
have relative L2 error <= 1e-3 and max-abs error <= 5e-3 * RMS against the
oracle's unrounded fp64 result; cases built so that every fp32 partial sum is
an exact integer are compared exactly (after the same final rounding).
"""
import os

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_L2, MAX_ABS_RMS = 1e-3, 5e-3


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_dequant_amd as m
    m.lib()
    return m


def dev():
    return torch.device("cuda:0")


def cu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def host(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64)


def assert_tol(y, y_exact, what=""):
    y = np.asarray(y, np.float64).ravel()
    e = np.asarray(y_exact, np.float64).ravel()
    rms = np.sqrt(np.mean(e ** 2))
    rel = np.linalg.norm(y - e) / max(np.linalg.norm(e), 1e-300)
    mx = np.max(np.abs(y - e)) / max(rms, 1e-300)
    print(f"{what}: rel_l2={rel:.3e} max_abs/rms={mx:.3e}")
    assert rel <= REL_L2, (what, rel)
    assert mx <= MAX_ABS_RMS, (what, mx)


U32 = 2.0 ** -24


def assert_fwd_bound(y, y_exact, abs_sum, n_terms, out="f16", what=""):
    """Element-wise forward error bound of an fp32 evaluation, then the output rounding.

    The kernels form every product exactly in fp32 and reach each output
    through at most n_terms + 8 rounded fp32 operations (the additions of any
    summation order, the scale and zero multiplies), so
      |v - y_exact| <= gamma_{n+8} * abs_sum,  gamma_n = n u / (1 - n u),
    abs_sum the sum of the magnitudes of the terms the kernel adds.  The
    stored y = round(v) adds u_out (|y_exact| + that) plus half the smallest
    subnormal of the output type.
    """
    y = np.asarray(y, np.float64)
    e = np.asarray(y_exact, np.float64)
    n = n_terms + 8
    g = n * U32 / (1 - n * U32)
    fwd = g * np.asarray(abs_sum, np.float64)
    uo, tiny = (2.0 ** -11, 2.0 ** -25) if out == "f16" else (U32, 2.0 ** -150)
    bound = fwd + uo * (np.abs(e) + fwd) + tiny
    ratio = np.max(np.abs(y - e) / bound)
    print(f"{what}: worst error / forward bound = {ratio:.3e}")
    assert ratio <= 1.0, (what, ratio)


# ================================================================== int8 ==

@pytest.mark.parametrize("M,K,N,G", [
    (1, 4096, 4096, 128),        # the headline GEMV
    (2, 4096, 4096, 128), (8, 4096, 4096, 128),  # the streaming lines the bench times
    (1, 256, 16, 128), (1, 384, 272, 128), (2, 512, 1024, 64), (3, 640, 528, 128),
    (4, 4096, 1040, 128), (5, 1024, 256, 32), (8, 2048, 4096, 128), (9, 768, 784, 128),
    (16, 256, 512, 256),
    (1, 8192, 512, 256),         # group scale folded after the quarter-wave sums, two chunks
    (1, 8192, 1024, 128),        # two chunks of 4096 rows, folded scales
    (1, 4608, 256, 512),         # a ragged second chunk (512 of 4096 rows)
    (1, 1152, 256, 96),          # group of 96 rows: a scale per piece, one row
    (1, 1536, 256, 384),         # group of 384 rows (not a power of two): a scale per piece
    (6, 8192, 512, 128),         # 8-row pass, activations restaged in LDS per chunk
    (7, 4224, 272, 64),          # 8-row pass, ragged chunk, scale per piece
    # One row and K = 4096 run the single-chunk form: larger groups (the
    # scale row of each 128-row block found by a shift), and panel counts
    # that are not a multiple of 16 (the plain workgroup-to-panel order).
    (1, 4096, 400, 256), (1, 4096, 1040, 1024), (1, 4096, 512, 4096), (1, 4096, 48, 2048),
])
def test_q8_group_vs_oracle(wq, M, K, N, G):
    d = synth.gen_q8_group(M, K, N, G, seed=1100 if (M, K, N) == (1, 4096, 4096) else 7 + M + K + N)
    Y = wq.gemm_q8_group(cu(d["X"]), wq.prepack_q8(cu(d["q"])), cu(d["scales"]), G)
    ref = oracle.gemm_q8_group(d["X"], d["q"], d["scales"], G)
    assert_tol(host(Y), ref, f"q8 {M}x{K}x{N} G{G}")
    A = np.abs(np.repeat(d["scales"].astype(np.float64), G, axis=0) * d["q"])
    assert_fwd_bound(host(Y), ref, np.abs(d["X"].astype(np.float64)) @ A, K, "f16", f"q8 {M}x{K}x{N} G{G}")


def test_q8_integer_exact(wq):
    # scale 1, small integer x: every fp32 partial sum is an exact integer.
    M, K, N, G = 3, 1024, 528, 128
    rng = np.random.default_rng(41)
    q = rng.integers(-127, 128, size=(K, N)).astype(np.int8)
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
    s = np.ones((K // G, N), np.float32)
    Y = host(wq.gemm_q8_group(cu(X), wq.prepack_q8(cu(q)), cu(s), G))
    ref = oracle.gemm_q8_group(X, q, s, G).astype(np.float16).astype(np.float64)
    assert np.array_equal(Y, ref)


def test_q8_output_rounding_ties(wq):
    # sum x*q = 2049 -> fp16 2048 and 2051 -> 2052 (round half to even).
    K, N, G = 128, 16, 128
    q = np.zeros((K, N), np.int8)
    x = np.zeros(K, np.float16)
    q[0, :], x[0] = 127, 16            # 2032 in every column
    q[2, 0], q[2, 1], x[2] = 17, 19, 1  # column 0: 2049, column 1: 2051
    s = np.ones((1, N), np.float32)
    y = host(wq.gemm_q8_group(cu(x), wq.prepack_q8(cu(q)), cu(s), G))
    assert y[0] == 2048 and y[1] == 2052


def test_q8_one_hot_rows(wq):
    K, N, G = 512, 272, 128
    d = synth.gen_q8_group(1, K, N, G, seed=42)
    packed = wq.prepack_q8(cu(d["q"]))
    for k in (0, 1, 127, 128, 300, 511):
        x = np.zeros(K, np.float16)
        x[k] = 1
        y = host(wq.gemm_q8_group(cu(x), packed, cu(d["scales"]), G))
        ref = (d["scales"][k // G].astype(np.float64) * d["q"][k]).astype(np.float16).astype(np.float64)
        assert np.array_equal(y, ref), k


def test_q8_deterministic_and_scale_exact(wq):
    d = synth.gen_q8_group(1, 4096, 4096, 128, seed=1100)
    X, q, s = cu(d["X"]), wq.prepack_q8(cu(d["q"])), cu(d["scales"])
    y0 = wq.gemm_q8_group(X, q, s, 128).clone()
    for _ in range(20):
        assert torch.equal(wq.gemm_q8_group(X, q, s, 128), y0)
    # Doubling x doubles every fp32 partial sum exactly; the final fp16
    # rounding commutes with the doubling wherever y is a normal fp16 value.
    y2 = wq.gemm_q8_group(X * 2, q, s, 128)
    normal = (y0.abs() >= 2.0 ** -14) & (y0.abs() < 2.0 ** 14)
    assert int(normal.sum()) > 4000
    assert torch.equal(y2[normal], (y0 * 2)[normal])


@pytest.mark.parametrize("K,N", [(4096, 4096), (4096, 11008), (11008, 4096), (1024, 8192), (96, 48)])
def test_unpack_q8_bit_exact(wq, K, N):
    d = synth.gen_q8_group(1, K, N, 32, seed=9 + K + N)
    codes = wq.unpack_q8(wq.prepack_q8(cu(d["q"])), K, N)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), d["q"])


def test_q8_wide_panels_and_long_k(wq):
    # Wide N, and K = 11008 (two chunks of 4096 rows and a ragged third).
    for (M, K, N) in ((1, 4096, 11008), (2, 11008, 4096), (3, 1024, 8192)):
        d = synth.gen_q8_group(M, K, N, 128, seed=M + K)
        Y = wq.gemm_q8_group(cu(d["X"]), wq.prepack_q8(cu(d["q"])), cu(d["scales"]), 128)
        assert_tol(host(Y), oracle.gemm_q8_group(d["X"], d["q"], d["scales"], 128), f"q8 {M}x{K}x{N}")


# From 33 rows of X on (groups a multiple of 64 rows) the int8 product runs
# as the tiled matrix-core GEMM: 32 x 128 output tiles, K in stages of 128
# rows, and K split over 2..8 workgroups while the tiles alone do not fill
# the GPU.
@pytest.mark.parametrize("M,K,N,G", [
    (33, 4096, 4096, 128),     # first row count on the tiled path: 8 K slices
    (48, 4096, 11008, 128),    # 8 slices, wide N
    (40, 4096, 4096, 64),      # groups of 64: two per stage
    (47, 2048, 4096, 256),     # groups of two stages: slices of 256 rows
    (56, 4096, 4096, 128),
    (64, 4096, 4096, 128),     # two row tiles, 8 slices
    (256, 4096, 4096, 128),    # 2 slices
    (36, 4160, 4096, 64),      # K not whole slices: no split
    (100, 1088, 4112, 64),     # ragged row and column tiles, 17 stages
    (64, 64, 128, 64),         # a single stage
    (40, 11008, 4096, 128),    # a ragged last stage (K = 86 stages of 128)
    (72, 4096, 8192, 128),     # wide N
    (33, 1152, 384, 192),      # groups of three stages
    (130, 512, 1024, 512),     # one group over all of K; three row tiles
])
def test_q8_gemm_tiles_vs_oracle(wq, M, K, N, G):
    d = synth.gen_q8_group(M, K, N, G, seed=31 + M + K + N)
    Y = wq.gemm_q8_group(cu(d["X"]), wq.prepack_q8(cu(d["q"])), cu(d["scales"]), G)
    assert_tol(host(Y), oracle.gemm_q8_group(d["X"], d["q"], d["scales"], G), f"q8 tiles {M}x{K}x{N} G{G}")


# Up to 32 rows of X the int8 product is one streaming matrix-core pass over
# the packed tiles: chains of 32-row steps per scale (groups of 32 .. 512
# rows a power of two, or one step per scale otherwise), X staged per 4096-row
# chunk (per 2048-row chunk above 16 rows, two 16-row tiles per step), the 8
# waves of a panel summed in LDS.
@pytest.mark.parametrize("M,K,N,G", [
    (9, 4096, 4096, 128),      # first row count past the 8-row operand tile rows
    (16, 4096, 11008, 128),    # the full 16-row pass, wide N
    (12, 224, 48, 32),         # K % 64 == 32: the last packed tile half padding; 3 panels
    (16, 1152, 272, 96),       # a scale per 32-row step (G not a power of two); 17 panels
    (13, 8192, 512, 4096),     # one chain per wave and chunk (G > 512), two chunks
    (11, 4608, 256, 512),      # a ragged second chunk (512 of 4096 rows)
    (10, 4224, 4112, 64),      # chains of two steps, a ragged chunk, N not a multiple of 256
    (15, 2048, 1024, 256),     # chains of eight steps
    # 17 .. 32 rows: two 16-row tiles per step, X staged per 2048-row chunk
    (17, 4096, 4096, 128),     # first row count past one tile; two chunks
    (32, 4096, 11008, 128),    # the full 32-row pass, wide N
    (24, 224, 48, 32),         # K % 64 == 32, a scale per step; 3 panels
    (32, 1152, 272, 96),       # G not a power of two; 17 panels
    (29, 8192, 512, 4096),     # eight-step chains inside one large group, four chunks
    (21, 4608, 256, 512),      # a ragged third chunk (512 of 2048 rows)
    (18, 4224, 4112, 64),      # chains of two steps, a ragged chunk, N not a multiple of 256
    (31, 2048, 1024, 256),     # eight-step chains of one group each
    (40, 1152, 512, 96),       # 40 rows with G = 96 (no tiled path): passes of 32 and 8
])
def test_q8_streaming_rows_vs_oracle(wq, M, K, N, G):
    d = synth.gen_q8_group(M, K, N, G, seed=301 + M + K + N)
    Y = wq.gemm_q8_group(cu(d["X"]), wq.prepack_q8(cu(d["q"])), cu(d["scales"]), G)
    ref = oracle.gemm_q8_group(d["X"], d["q"], d["scales"], G)
    assert_tol(host(Y), ref, f"q8 streaming {M}x{K}x{N} G{G}")
    A = np.abs(np.repeat(d["scales"].astype(np.float64), G, axis=0) * d["q"])
    assert_fwd_bound(host(Y), ref, np.abs(d["X"].astype(np.float64)) @ A, K, "f16",
                     f"q8 streaming {M}x{K}x{N} G{G}")


@pytest.mark.parametrize("M,K,N,G", [(80, 1024, 400, 128), (12, 2048, 1024, 128),
                                     (16, 2048, 1024, 64), (3, 4160, 272, 32),
                                     (24, 2048, 1024, 64), (32, 4160, 272, 32)])
def test_q8_gemm_integer_exact_and_deterministic(wq, M, K, N, G):
    # Scales 1 and small integer X on the tiled path (80 rows) and the
    # streaming passes (3..32 rows): every fp32 partial sum is an exact
    # integer, so the result is bit-exact; repeated calls agree.
    rng = np.random.default_rng(43)
    q = rng.integers(-127, 128, size=(K, N)).astype(np.int8)
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
    s = np.ones((K // G, N), np.float32)
    Xd, P, Sd = cu(X), wq.prepack_q8(cu(q)), cu(s)
    Y = wq.gemm_q8_group(Xd, P, Sd, G)
    ref = oracle.gemm_q8_group(X, q, s, G).astype(np.float16).astype(np.float64)
    assert np.array_equal(host(Y), ref)
    for _ in range(5):
        assert torch.equal(wq.gemm_q8_group(Xd, P, Sd, G), Y)


def test_q8_split_k_workspace_contents_do_not_matter(wq):
    # The K slices' partial tiles overwrite the workspace: garbage in it, or
    # a larger one, changes nothing, and two calls in a row (the second
    # smaller) agree with fresh ones.
    d = synth.gen_q8_group(40, 4096, 4096, 128, seed=91)
    X, P, Sd = cu(d["X"]), wq.prepack_q8(cu(d["q"])), cu(d["scales"])
    need = wq.workspace_bytes(wq.WQ_OP_Q8G, 40, 4096, 4096)
    assert need == 8 * 40 * 4096 * 4
    ws = torch.full((need + 4096,), 0x7F, dtype=torch.uint8, device=dev())
    Y0 = wq.gemm_q8_group(X, P, Sd, 128)
    assert torch.equal(wq.gemm_q8_group(X, P, Sd, 128, ws=ws), Y0)
    Y1 = wq.gemm_q8_group(X[:10], P, Sd, 128, ws=ws)
    assert torch.equal(Y1, wq.gemm_q8_group(X[:10], P, Sd, 128))
    assert_tol(host(Y0), oracle.gemm_q8_group(d["X"], d["q"], d["scales"], 128), "q8 split 40")
    assert_tol(host(Y1), oracle.gemm_q8_group(d["X"][:10], d["q"], d["scales"], 128), "q8 split 10")


def test_q8_gemm_rows_match_single_row_calls(wq):
    # Row m of the tiled product against the streaming kernel on row m alone:
    # both within the bar of the oracle, and close to each other.
    M, K, N, G = 48, 2048, 1024, 128
    d = synth.gen_q8_group(M, K, N, G, seed=77)
    P, Sd = wq.prepack_q8(cu(d["q"])), cu(d["scales"])
    Y = host(wq.gemm_q8_group(cu(d["X"]), P, Sd, G))
    for m in (0, 17, 47):
        y1 = host(wq.gemm_q8_group(cu(d["X"][m:m + 1]), P, Sd, G))
        ref = oracle.gemm_q8_group(d["X"][m:m + 1], d["q"], d["scales"], G)
        assert_tol(Y[m], ref, f"tiled row {m}")
        assert_tol(y1, ref, f"streaming row {m}")


def test_q8_gemm_full_size_sampled_rows(wq):
    # M = 512, K = N = 4096, group 128: the int8 workload of the fused-kernel
    # page.  All rows on the GPU; the oracle on a sample of rows (row m of Y
    # depends on row m of X only).
    M, K, N, G = 512, 4096, 4096, 128
    d = synth.gen_q8_group(M, K, N, G, seed=1500)
    Y = host(wq.gemm_q8_group(cu(d["X"]), wq.prepack_q8(cu(d["q"])), cu(d["scales"]), G))
    rows = [0, 1, 63, 64, 127, 200, 255, 256, 383, 447, 510, 511]
    ref = oracle.gemm_q8_group(d["X"][rows], d["q"], d["scales"], G)
    assert_tol(Y[rows], ref, "q8 512x4096x4096 sampled rows")
    assert np.all(np.isfinite(Y))


# ============================================ separated form (comparator) ==

@pytest.mark.parametrize("K,N,G", [(4096, 4096, 128), (1024, 4112, 64), (96, 48, 32), (11008, 4096, 128)])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_dequant_q8_bit_exact(wq, K, N, G, dt):
    # The materialised weight: one fp32 multiply per weight (then one fp16
    # rounding): bit for bit the oracle's.
    d = synth.gen_q8_group(1, K, N, G, seed=41 + K + N)
    W = wq.dequant_q8_group(cu(d["q"]), cu(d["scales"]), G,
                            torch.float32 if dt == "f32" else torch.float16)
    ref = oracle.materialize_q8_group(d["q"], d["scales"], G, dt)
    got = W.cpu().numpy()
    bits = np.uint32 if dt == "f32" else np.uint16
    assert np.array_equal(got.view(bits), ref.view(bits))


def test_dequant_q8_worked_example(wq):
    # tests/golden/q8_materialize_worked.txt on the GPU: fp32 product rounded
    # down to an fp16 tie, then to even (16 columns: one row of the kernel).
    for name, sc, q, b32, b16 in read_golden("q8_materialize_worked.txt"):
        qq = np.full((32, 16), int(q), np.int8)
        s = np.full((1, 16), np.float32(int(sc) * 2.0 ** -26), np.float32)
        w32 = wq.dequant_q8_group(cu(qq), cu(s), 32, torch.float32).cpu().numpy()
        w16 = wq.dequant_q8_group(cu(qq), cu(s), 32, torch.float16).cpu().numpy()
        assert np.all(w32.view(np.uint32) == int(b32, 16)), name
        assert np.all(w16.view(np.uint16) == int(b16, 16)), name


def test_separated_form_vs_oracle(wq):
    # The unfused comparator at the fused-kernel page's workload (M = 512,
    # K = N = 4096, group 128): dequantise to fp16, then a library GEMM
    # (fp32 accumulation); the oracle on a sample of rows.  The fp16 weight
    # adds one rounding per weight (relative 2^-11), within the bar.
    M, K, N, G = 512, 4096, 4096, 128
    d = synth.gen_q8_group(M, K, N, G, seed=1500)
    W16 = wq.dequant_q8_group(cu(d["q"]), cu(d["scales"]), G, torch.float16)
    Y = torch.matmul(cu(d["X"]), W16)
    rows = [0, 1, 255, 256, 511]
    assert_tol(host(Y)[rows], oracle.gemm_q8_group(d["X"][rows], d["q"], d["scales"], G),
               "separated fp16 512x4096x4096")
    W32 = wq.dequant_q8_group(cu(d["q"]), cu(d["scales"]), G, torch.float32)
    Y32 = torch.matmul(cu(d["X"]).float(), W32)
    assert_tol(host(Y32)[rows], oracle.gemm_q8_group(d["X"][rows], d["q"], d["scales"], G),
               "separated fp32 512x4096x4096")


# ================================================================= 3-bit ==

@pytest.mark.parametrize("K,N", [(1024, 1024), (4096, 4096), (4096, 11008), (11008, 4096), (96, 20)])
def test_unpack_q3_bit_exact(wq, K, N):
    d = synth.gen_q3(K, N, seed=5 + K + N, dtype="f16")
    codes = wq.unpack_q3(wq.prepack_q3(cu(d["qweight"]), K), K, N)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy().astype(np.int64), oracle.unpack_q3(d["qweight"]))


@pytest.mark.parametrize("K,N,dt,seed", [
    (1024, 1024, "f32", 1000),                     # the 3-bit fp32 matvec
    (4096, 4096, "f16", 1200), (4096, 11008, "f16", 1201), (11008, 4096, "f16", 1202),
    (32, 4, "f32", 3), (96, 260, "f16", 4), (1056, 516, "f32", 5), (2080, 1028, "f16", 6),
])
def test_q3_vs_oracle(wq, K, N, dt, seed):
    d = synth.gen_q3(K, N, seed=seed, dtype=dt)
    y = wq.matvec_q3(cu(d["x"]), wq.prepack_q3(cu(d["qweight"]), K), cu(d["scales"]), cu(d["zeros"]))
    ref = oracle.matvec_q3(d["x"], d["qweight"], d["scales"], d["zeros"])
    assert_tol(host(y), ref, f"q3 {dt} {K}x{N}")
    # the kernel adds s * x * q and z * x terms (the zero is applied through sum x)
    ax = np.abs(d["x"].astype(np.float64))
    abs_sum = (ax @ d["codes"].astype(np.float64)) * np.abs(d["scales"].astype(np.float64)) \
        + ax.sum() * np.abs(d["zeros"].astype(np.float64))
    assert_fwd_bound(host(y), ref, abs_sum, K, dt, f"q3 {dt} {K}x{N}")


@pytest.mark.parametrize("K,N,dt", [
    (64, 8208, "f16"),     # 2052 four-column panels: runs of 8 panels over 257 workgroups
    (128, 3076, "f32"),    # 769 panels: runs of 3 and 4
    (32768, 64, "f16"),    # x fills 64 KB of LDS next to the per-panel partial sums
    (16384, 132, "f32"),
])
def test_q3_long_runs_and_long_k(wq, K, N, dt):
    d = synth.gen_q3(K, N, seed=K + N, dtype=dt)
    y = wq.matvec_q3(cu(d["x"]), wq.prepack_q3(cu(d["qweight"]), K), cu(d["scales"]), cu(d["zeros"]))
    ref = oracle.matvec_q3(d["x"], d["qweight"], d["scales"], d["zeros"])
    assert_tol(host(y), ref, f"q3 {dt} {K}x{N}")


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_q3_integer_exact_and_zero_codes(wq, dt):
    K, N = 1024, 516
    rng = np.random.default_rng(51)
    npdt = np.float32 if dt == "f32" else np.float16
    codes = rng.integers(0, 8, size=(K, N))
    z = rng.integers(0, 8, size=N).astype(npdt)
    x = rng.integers(-3, 4, size=K).astype(npdt)
    s = np.ones(N, npdt)
    y = host(wq.matvec_q3(cu(x), wq.prepack_q3(cu(synth.pack_q3(codes)), K), cu(s), cu(z)))
    ref = oracle.matvec_q3(x, synth.pack_q3(codes), s, z).astype(npdt).astype(np.float64)
    assert np.array_equal(y, ref)
    # all-zero codes: y = -zero * sum(x)
    zero_w = wq.prepack_q3(cu(synth.pack_q3(np.zeros((K, N), np.int64))), K)
    y0 = host(wq.matvec_q3(cu(x), zero_w, cu(s), cu(z)))
    assert np.array_equal(y0, (-z.astype(np.float64) * x.astype(np.float64).sum()).astype(npdt).astype(np.float64))


def test_q3_one_hot_rows(wq):
    K, N = 256, 260
    d = synth.gen_q3(K, N, seed=52, dtype="f32")
    packed = wq.prepack_q3(cu(d["qweight"]), K)
    for k in (0, 6, 10, 21, 31, 32, 100, 255):
        x = np.zeros(K, np.float32)
        x[k] = 1
        y = host(wq.matvec_q3(cu(x), packed, cu(d["scales"]), cu(d["zeros"])))
        ref = d["scales"].astype(np.float64) * d["codes"][k] - d["zeros"].astype(np.float64)
        assert np.allclose(y, ref, rtol=1e-6, atol=1e-7), k


# ================================================================= 4-bit ==

def _q4_abs_sum(X, qweight, scales, zeros, g_idx, G, unpack=None):
    """sum_k |x| * s * (u + |zero|): the magnitudes of the terms the 4-bit and
    2-bit kernels add (x * u * s, and the zero, 8 for symmetric codes, times
    s * sum x)."""
    u = (unpack or oracle.unpack_u4)(qweight).astype(np.float64)
    K = u.shape[0]
    g = np.asarray(g_idx) if g_idx is not None else np.arange(K) // G
    s = np.abs(scales.astype(np.float64))[g]
    z = np.full_like(s, 8.0) if zeros is None else np.abs(zeros.astype(np.float64))[g]
    return np.abs(np.atleast_2d(X).astype(np.float64)) @ (s * (u + z))


@pytest.mark.parametrize("act", [True, False])
def test_unpack_q4_bit_exact(wq, act):
    K, N, G = 4096, 11008, 128
    d = synth.gen_q4_group(1, K, N, G, seed=1300, act_order=act)
    packed, perm = wq.prepare_q4(cu(d["qweight"]), d["g_idx"] if act else None, G)
    codes = wq.unpack_q4(packed, K, N, G, perm)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy().astype(np.int64), oracle.unpack_q4(d["qweight"]))


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_q4_act_order_headline(wq, M):
    K, N, G = 4096, 11008, 128
    d = synth.gen_q4_group(M, K, N, G, seed=1300, act_order=True)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"], G)
    Y = wq.gemm_q4_group(cu(d["X"]), packed, cu(d["scales"]), G)
    ref = oracle.gemm_q4_group(d["X"], d["qweight"], d["scales"], d["g_idx"], G)
    assert_tol(host(Y), ref, f"q4 M{M}")
    assert_fwd_bound(host(Y), ref, _q4_abs_sum(d["X"], d["qweight"], d["scales"], None, d["g_idx"], G),
                     K, "f16", f"q4 M{M}")


@pytest.mark.parametrize("M,K,N,G,act", [
    (1, 128, 4, 32, True), (3, 384, 260, 64, True), (5, 1024, 1028, 128, False),
    (9, 512, 516, 128, True), (2, 2048, 256, 32, False), (16, 256, 64, 128, True),
    (1, 4096, 4096, 128, True), (4, 11008, 4096, 128, True), (1, 544, 1024, 32, True),
    (2, 2048, 264, 256, True), (1, 4096, 1024, 512, False),   # groups spanning 2 and 4 blocks
])
def test_q4_small_ragged(wq, M, K, N, G, act):
    d = synth.gen_q4_group(M, K, N, G, seed=60 + M + K, act_order=act)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"] if act else None, G)
    Y = wq.gemm_q4_group(cu(d["X"]), packed, cu(d["scales"]), G)
    ref = oracle.gemm_q4_group(d["X"], d["qweight"], d["scales"], d["g_idx"], G)
    assert_tol(host(Y), ref, f"q4 {M}x{K}x{N} G{G} act={act}")


def test_q4_one_hot_act_order(wq):
    K, N, G = 512, 260, 128
    d = synth.gen_q4_group(1, K, N, G, seed=61, act_order=True)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"], G)
    for k in (0, 1, 5, 200, 511):
        x = np.zeros(K, np.float16)
        x[k] = 1
        y = host(wq.gemm_q4_group(cu(x), packed, cu(d["scales"]), G))
        ref = (d["scales"][d["g_idx"][k]].astype(np.float64) * d["codes"][k]).astype(np.float16)
        assert np.array_equal(y, ref.astype(np.float64)), k


def test_q4_integer_exact(wq):
    M, K, N, G = 4, 1024, 516, 128
    rng = np.random.default_rng(62)
    q = rng.integers(-8, 8, size=(K, N))
    g_idx = rng.permutation(np.repeat(np.arange(K // G), G)).astype(np.int32)
    s = np.ones((K // G, N), np.float16)
    X = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    qw = synth.pack_q4(q + 8)
    packed, _ = wq.prepare_q4(cu(qw), g_idx, G)
    Y = host(wq.gemm_q4_group(cu(X), packed, cu(s), G))
    ref = oracle.gemm_q4_group(X, qw, s, g_idx, G).astype(np.float16).astype(np.float64)
    assert np.array_equal(Y, ref)


# ---------------------------- 4-bit above 8 rows: the packed weight read once

@pytest.mark.parametrize("zp", [False, True])
@pytest.mark.parametrize("M", [16, 32, 64])
def test_q4_tiled_layer_shape(wq, M, zp):
    # K = 4096, N = 11008, group 128, act-order, with and without zero points.
    K, N, G = 4096, 11008, 128
    if zp:
        d = synth.gen_q4_zp(M, K, N, G, seed=synth.SEEDS["q4_zp"] + M, act_order=True)
        packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"], G)
        Y = wq.gemm_q4_group_zp(cu(d["X"]), packed, cu(d["scales"]), cu(d["zeros"]), G)
        ref = oracle.gemm_q4_zp(d["X"], d["qweight"], d["scales"], d["zeros"], d["g_idx"], G)
    else:
        d = synth.gen_q4_group(M, K, N, G, seed=1300, act_order=True)
        packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"], G)
        Y = wq.gemm_q4_group(cu(d["X"]), packed, cu(d["scales"]), G)
        ref = oracle.gemm_q4_group(d["X"], d["qweight"], d["scales"], d["g_idx"], G)
    y = host(Y)
    assert_tol(y, ref, f"q4 tiled M{M} zp={zp}")
    assert_fwd_bound(y, ref, _q4_abs_sum(d["X"], d["qweight"], d["scales"], d.get("zeros") if zp else None,
                                         d["g_idx"], G), K, "f16", f"q4 tiled M{M} zp={zp}")


@pytest.mark.parametrize("M,K,N,G,act,zp", [
    (9, 4096, 11008, 128, True, False),    # 9 rows in one 16-row tile
    (17, 2048, 4100, 64, True, True),      # two tiles; ragged last panel
    (33, 4160, 1040, 32, True, False),     # K = 32.5 blocks (padded to 4224), groups of 32
    (40, 4160, 1040, 32, True, True),      # groups of 32 with zero points
    (47, 1024, 256, 256, False, True),     # groups spanning two blocks
    (63, 8192, 528, 512, True, False),     # groups spanning four blocks, long K
    (65, 1024, 1024, 128, True, False),    # 64 + 1 rows: two launches over the weight
    (130, 512, 64, 128, True, True),       # three launches, four panels
    (12, 128, 4, 32, True, True),          # one block, one panel of four columns
])
def test_q4_tiled_ragged(wq, M, K, N, G, act, zp):
    if zp:
        d = synth.gen_q4_zp(M, K, N, G, seed=90 + M + K, act_order=act)
    else:
        d = synth.gen_q4_group(M, K, N, G, seed=90 + M + K, act_order=act)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"] if act else None, G)
    if zp:
        Y = wq.gemm_q4_group_zp(cu(d["X"]), packed, cu(d["scales"]), cu(d["zeros"]), G)
        ref = oracle.gemm_q4_zp(d["X"], d["qweight"], d["scales"], d["zeros"], d["g_idx"], G)
    else:
        Y = wq.gemm_q4_group(cu(d["X"]), packed, cu(d["scales"]), G)
        ref = oracle.gemm_q4_group(d["X"], d["qweight"], d["scales"], d["g_idx"], G)
    y = host(Y)
    what = f"q4 tiled {M}x{K}x{N} G{G} act={act} zp={zp}"
    assert_tol(y, ref, what)
    assert_fwd_bound(y, ref, _q4_abs_sum(d["X"], d["qweight"], d["scales"], d["zeros"] if zp else None,
                                         d["g_idx"], G), K, "f16", what)


@pytest.mark.parametrize("M", [1, 9, 40])
def test_q4_longest_k(wq, M):
    # K = 32768, the longest K the packed row tables allow (uint16 rows):
    # the small-M kernel at one row, the tiled kernel at 9 and 40 rows
    # (one tile; three tiles in two row groups), act-order.
    K, N, G = 32768, 64, 128
    d = synth.gen_q4_group(M, K, N, G, seed=1330 + M, act_order=True)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"], G)
    y = host(wq.gemm_q4_group(cu(d["X"]), packed, cu(d["scales"]), G))
    ref = oracle.gemm_q4_group(d["X"], d["qweight"], d["scales"], d["g_idx"], G)
    what = f"q4 K=32768 M{M}"
    assert_tol(y, ref, what)
    assert_fwd_bound(y, ref, _q4_abs_sum(d["X"], d["qweight"], d["scales"], None, d["g_idx"], G), K,
                     "f16", what)


def test_q4_tiled_integer_exact_and_one_hot(wq):
    # Scales 1 and small integer X: every fp32 partial sum is an exact
    # integer, so Y is the oracle's value after one fp16 rounding.  Then one
    # row of X per original row k (one-hot): row m of Y is scale[g_idx[k]] *
    # q[k], which pins the row order through the act-order table.
    M, K, N, G = 24, 1024, 64, 128
    rng = np.random.default_rng(97)
    d = synth.gen_q4_group(1, K, N, G, seed=98, act_order=True)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"], G)
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
    ones = np.ones_like(d["scales"])
    Y = host(wq.gemm_q4_group(cu(X), packed, cu(ones), G))
    ref = oracle.gemm_q4_group(X, d["qweight"], ones, d["g_idx"], G).astype(np.float16).astype(np.float64)
    assert np.array_equal(Y, ref)
    rows = rng.choice(K, size=M, replace=False)
    X1 = np.zeros((M, K), np.float16)
    X1[np.arange(M), rows] = 1
    Y1 = host(wq.gemm_q4_group(cu(X1), packed, cu(d["scales"]), G))
    q = oracle.unpack_q4(d["qweight"])
    expect = (d["scales"].astype(np.float64)[d["g_idx"][rows]] * q[rows]).astype(np.float16).astype(np.float64)
    assert np.array_equal(Y1, expect)


def test_q4_tiled_matches_row_by_row(wq):
    # Rows of a 40-row call equal the same rows computed alone (the small-M
    # kernel, one row per call) within the tolerance; and a call reusing a
    # workspace with garbage in it gives the same bits as a fresh one.
    M, K, N, G = 40, 2048, 1024, 128
    d = synth.gen_q4_group(M, K, N, G, seed=99, act_order=True)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"], G)
    X, S = cu(d["X"]), cu(d["scales"])
    Y = wq.gemm_q4_group(X, packed, S, G)
    ws = torch.randint(-128, 127, (wq.workspace_bytes(wq.WQ_OP_Q4G, M, K, N) + 64,), dtype=torch.int8,
                       device=dev())
    assert torch.equal(wq.gemm_q4_group(X, packed, S, G, ws=ws), Y)
    assert torch.equal(wq.gemm_q4_group(X, packed, S, G, ws=ws), Y)
    ref = oracle.gemm_q4_group(d["X"], d["qweight"], d["scales"], d["g_idx"], G)
    for m in (0, 17, 39):
        ym = host(wq.gemm_q4_group(X[m:m + 1].contiguous(), packed, S, G))
        assert_tol(ym, ref[m:m + 1], f"row {m} alone")
    assert_tol(host(Y), ref, "40 rows")


# ====================================================== asymmetric 4-bit ==

@pytest.mark.parametrize("M,K,N,G,act", [
    (1, 4096, 11008, 128, False),   # AWQ-style layer shape, no act-order
    (1, 4096, 4096, 64, False),     # group 64
    (4, 2048, 1024, 32, False),     # group 32: four scale and zero loads per block
    (8, 1024, 528, 128, False),
    (3, 1024, 260, 128, True),      # zeros with an act-order row table; ragged N
    (12, 512, 1028, 128, False),    # two row chunks (8 + 4)
    (3, 2048, 132, 256, True),      # a group spans two blocks
])
def test_q4_zp_vs_oracle(wq, M, K, N, G, act):
    d = synth.gen_q4_zp(M, K, N, G, seed=synth.SEEDS["q4_zp"] + K + N, act_order=act)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"] if act else None, G)
    Y = wq.gemm_q4_group_zp(cu(d["X"]), packed, cu(d["scales"]), cu(d["zeros"]), G)
    ref = oracle.gemm_q4_zp(d["X"], d["qweight"], d["scales"], d["zeros"], d["g_idx"], G)
    assert_tol(host(Y), ref, f"q4 zp {M}x{K}x{N} G{G} act={act}")
    assert_fwd_bound(host(Y), ref, _q4_abs_sum(d["X"], d["qweight"], d["scales"], d["zeros"], d["g_idx"], G),
                     K, "f16", f"q4 zp {M}x{K}x{N}")


def test_q4_zp_integer_exact_gpu(wq):
    # Scales 1, integer zeros and small integer X: every fp32 partial sum is an
    # exact integer, so the result equals the oracle's after one fp16 rounding.
    rng = np.random.default_rng(65)
    M, K, N, G = 2, 1024, 64, 128
    u = rng.integers(0, 16, size=(K, N))
    z = rng.integers(0, 16, size=(K // G, N)).astype(np.float16)
    s = np.ones((K // G, N), np.float16)
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
    qw = synth.pack_q4(u)
    packed, _ = wq.prepare_q4(cu(qw), None, G)
    Y = host(wq.gemm_q4_group_zp(cu(X), packed, cu(s), cu(z), G))
    ref = oracle.gemm_q4_zp(X, qw, s, z, None, G).astype(np.float16).astype(np.float64)
    assert np.array_equal(Y, ref)


def test_q4_zp_zero_eight_matches_symmetric_kernel(wq):
    # The same packed weight through both entry points: zeros of 8 reproduce
    # the symmetric product bit for bit (same kernel, same order of sums).
    d = synth.gen_q4_group(4, 2048, 512, 128, seed=66, act_order=True)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"], 128)
    X, S = cu(d["X"]), cu(d["scales"])
    z8 = torch.full_like(S, 8.0)
    assert torch.equal(wq.gemm_q4_group_zp(X, packed, S, z8, 128), wq.gemm_q4_group(X, packed, S, 128))


# ================================================================= 2-bit ==

@pytest.mark.parametrize("K,N,G,act", [(4096, 11008, 128, True), (4096, 11008, 128, False)])
def test_unpack_q2_bit_exact(wq, K, N, G, act):
    d = synth.gen_q2_zp(1, K, N, G, seed=71 + int(act), act_order=act)
    packed, perm = wq.prepare_q2(cu(d["qweight"]), d["g_idx"] if act else None, G)
    u = wq.unpack_q2(packed, K, N, G, perm)
    torch.cuda.synchronize()
    assert np.array_equal(u.cpu().numpy().astype(np.int64), oracle.unpack_u2(d["qweight"]))


@pytest.mark.parametrize("M,K,N,G,act", [
    (1, 4096, 11008, 128, True), (2, 4096, 11008, 128, False), (4, 4096, 11008, 64, True),
    (8, 4096, 11008, 256, False), (1, 4096, 4096, 32, True),
    (3, 544, 20, 32, False),       # ragged: a partial 256-row block, N % 16 != 0
    (5, 1280, 132, 128, True),     # two groups per block, 9 panels
    (1, 8192, 64, 512, False),     # a group spans two blocks
])
def test_q2_vs_oracle(wq, M, K, N, G, act):
    d = synth.gen_q2_zp(M, K, N, G, seed=synth.SEEDS["q2_zp"] + K + N + G, act_order=act)
    packed, _ = wq.prepare_q2(cu(d["qweight"]), d["g_idx"] if act else None, G)
    Y = wq.gemm_q2_group_zp(cu(d["X"]), packed, cu(d["scales"]), cu(d["zeros"]), G)
    ref = oracle.gemm_q2_zp(d["X"], d["qweight"], d["scales"], d["zeros"], d["g_idx"], G)
    assert_tol(host(Y), ref, f"q2 {M}x{K}x{N} G{G} act={act}")
    assert_fwd_bound(host(Y), ref, _q4_abs_sum(d["X"], d["qweight"], d["scales"], d["zeros"], d["g_idx"], G,
                                               unpack=oracle.unpack_u2), K, "f16", f"q2 {M}x{K}x{N}")


def test_q2_integer_exact_and_one_hot(wq):
    # Scales 1, integer zeros and small integer X: every fp32 partial sum is an
    # exact integer, so the result equals the oracle's after one fp16 rounding.
    rng = np.random.default_rng(72)
    M, K, N, G = 3, 1024, 48, 64
    u = rng.integers(0, 4, size=(K, N))
    z = rng.integers(0, 4, size=(K // G, N)).astype(np.float16)
    s = np.ones((K // G, N), np.float16)
    X = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    g_idx = rng.permutation(np.repeat(np.arange(K // G), G)).astype(np.int32)
    qw = synth.pack_q2(u)
    packed, _ = wq.prepare_q2(cu(qw), g_idx, G)
    Y = host(wq.gemm_q2_group_zp(cu(X), packed, cu(s), cu(z), G))
    ref = oracle.gemm_q2_zp(X, qw, s, z, g_idx, G).astype(np.float16).astype(np.float64)
    assert np.array_equal(Y, ref)
    # One-hot rows: y[n] = u[k, n] - zero[g_idx[k], n] exactly, row by row.
    for k in (0, 7, 8, 15, 31, 32, 255, 256, 700, 1023):
        x = np.zeros((1, K), np.float16)
        x[0, k] = 1
        y = host(wq.gemm_q2_group_zp(cu(x), packed, cu(s), cu(z), G))[0]
        assert np.array_equal(y, u[k].astype(np.float64) - z[g_idx[k]].astype(np.float64)), k


def test_q2_deterministic(wq):
    d = synth.gen_q2_zp(2, 4096, 1024, 128, seed=73, act_order=True)
    packed, _ = wq.prepare_q2(cu(d["qweight"]), d["g_idx"], 128)
    X, S, Z = cu(d["X"]), cu(d["scales"]), cu(d["zeros"])
    first = wq.gemm_q2_group_zp(X, packed, S, Z, 128)
    for _ in range(20):
        assert torch.equal(wq.gemm_q2_group_zp(X, packed, S, Z, 128), first)


# ================================================================== W8A8 ==

def _w8a8_check(wq, d):
    Y, Xq, Sx, acc = wq.gemm_w8a8(cu(d["X"]), cu(d["Wq"]), cu(d["Sw"]), want_acc=True)
    torch.cuda.synchronize()
    r = oracle.gemm_w8a8(d["X"], d["Wq"], d["Sw"])
    assert np.array_equal(Xq.cpu().numpy(), r["Xq"])
    assert np.array_equal(Sx.cpu().numpy().view(np.uint32), r["Sx"].view(np.uint32))
    assert np.array_equal(acc.cpu().numpy(), r["acc"])
    yb = Y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(yb, r["y_bits"])
    return Y, r


@pytest.mark.parametrize("M,K,N", [(1, 64, 16), (17, 192, 80), (128, 512, 256), (130, 256, 528),
                                   (256, 1024, 1040), (64, 640, 64), (300, 4160, 208),
                                   (3, 2048, 4096), (600, 2048, 144), (1100, 512, 2048)])
def test_w8a8_small_bit_exact(wq, M, K, N):
    # K split into 1 to 8 slices (workspace partials summed by the second
    # kernel, or the rescale in the GEMM itself), ragged M, N and K tiles.
    _w8a8_check(wq, synth.gen_w8a8(M, K, N, seed=70 + M + K + N))


def test_w8a8_workspace_contents_do_not_matter(wq):
    # The partial tiles overwrite the workspace: garbage in it, a larger one,
    # or one reused by the previous call give the same bits.
    d = synth.gen_w8a8(256, 4096, 1024, seed=77)
    need = wq.workspace_bytes(wq.WQ_OP_W8A8, 256, 4096, 1024)
    assert need > 0
    ws = torch.randint(-128, 127, (need + 4096,), dtype=torch.int8, device=dev())
    X, Wq, Sw = cu(d["X"]), cu(d["Wq"]), cu(d["Sw"])
    ref = wq.gemm_w8a8(X, Wq, Sw, want_acc=True)
    for _ in range(2):
        got = wq.gemm_w8a8(X, Wq, Sw, want_acc=True, ws=ws)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)


@pytest.mark.parametrize("M,K,N", [(256, 8192, 8192), (64, 8192, 4096)])
def test_w8a8_alternating_inputs_share_a_workspace(wq, M, K, N):
    # Two inputs in turn on one workspace, six calls each: the sum of the K
    # slices must take this call's partials, never the previous call's (which
    # hold the other input's values).
    ds = [synth.gen_w8a8(M, K, N, seed=1410 + i) for i in range(2)]
    args = [(cu(d["X"]), cu(d["Wq"]), cu(d["Sw"])) for d in ds]
    refs = [wq.gemm_w8a8(*a, want_acc=True) for a in args]
    ws = torch.zeros(wq.workspace_bytes(wq.WQ_OP_W8A8, M, K, N), dtype=torch.int8, device=dev())
    for it in range(12):
        got = wq.gemm_w8a8(*args[it % 2], want_acc=True, ws=ws)
        for a, b in zip(refs[it % 2], got):
            assert torch.equal(a, b), f"call {it}"
    r = oracle.gemm_w8a8(ds[1]["X"], ds[1]["Wq"], ds[1]["Sw"])
    assert np.array_equal(refs[1][3].cpu().numpy(), r["acc"])


def test_w8a8_headline_bit_exact(wq):
    Y, r = _w8a8_check(wq, synth.gen_w8a8(256, 8192, 8192, seed=1400))
    # reported, not gated: distance of the bf16 result to the unrounded product
    y = Y.float().cpu().numpy().astype(np.float64)
    e = r["y_exact"]
    print("w8a8 bf16 vs exact: rel_l2=%.3e" % (np.linalg.norm(y - e) / np.linalg.norm(e)))


def test_w8a8_ties_and_zero_row(wq):
    K, N = 64, 16
    X = np.zeros((3, K), np.float32)
    X[0, 0], X[0, 1] = 127.0, 1.0        # Sx = 1; Xq = [127, 1, 0...]
    X[1, :4] = [127.0, 2.5, -3.5, 0.5]   # halves round to even: 2, -4, 0
    Wq = np.zeros((N, K), np.int8)
    Wq[0, 0], Wq[0, 1] = 2, 3            # acc = 257 -> bf16 256
    Wq[1, 0], Wq[1, 1] = 2, 5            # acc = 259 -> bf16 260
    Wq[2, 0], Wq[2, 1] = 4, 6            # acc = 514 -> 512
    Wq[3, 0], Wq[3, 1] = 4, 10           # acc = 518 -> 520
    Sw = np.ones(N, np.float32)
    Y, Xq, Sx, acc = wq.gemm_w8a8(cu(X), cu(Wq), cu(Sw), want_acc=True)
    torch.cuda.synchronize()
    y = Y.float().cpu().numpy()
    assert y[0, :4].tolist() == [256.0, 260.0, 512.0, 520.0]
    assert Xq.cpu().numpy()[1, :4].tolist() == [127, 2, -4, 0]
    assert Sx.cpu().numpy()[2] == 0 and np.all(Xq.cpu().numpy()[2] == 0) and np.all(y[2] == 0)


def test_w8a8_longest_k_int32_range(wq):
    # K = 133120, the largest multiple of 64 with K * 127 * 127 < 2^31.  Row
    # 0 of X and every weight code sit at +127, so acc = K * 127^2 =
    # 2,147,092,480: the int32 accumulators and the K-slice partials end
    # within 0.02% of their range, and must still equal the oracle's exact
    # sums; row 1 is random.
    K, N = 133120, 32
    assert K * 127 * 127 < 2**31 and (K + 64) * 127 * 127 >= 2**31
    rng = np.random.default_rng(1430)
    X = np.stack([np.ones(K, np.float32), rng.standard_normal(K).astype(np.float32)])
    Wq = np.full((N, K), 127, np.int8)
    Wq[N // 2:] = rng.integers(-127, 128, size=(N - N // 2, K)).astype(np.int8)
    Sw = rng.uniform(0.5, 2.0, N).astype(np.float32)
    Y, Xq, Sx, acc = wq.gemm_w8a8(cu(X), cu(Wq), cu(Sw), want_acc=True)
    torch.cuda.synchronize()
    r = oracle.gemm_w8a8(X, Wq, Sw)
    a = acc.cpu().numpy()
    assert int(a[0, 0]) == K * 127 * 127
    assert np.array_equal(Xq.cpu().numpy(), r["Xq"])
    assert np.array_equal(a, r["acc"])
    assert np.array_equal(Y.view(torch.int16).cpu().numpy().view(np.uint16), r["y_bits"])


def test_w8a8_quantiser_division_at_ties_and_extreme_scales(wq):
    # The quantiser divides by the row's Sx with one reciprocal per row and
    # two fmas per element, which must give the IEEE quotient bit for bit.
    # Rows with Sx from 2^-130 (subnormal) to 2^120 (below 2^-100 the plain
    # division: near 2^-126 the remainder of the shortcut underflows), and
    # entries whose quotients are exact halves and one ulp either side of
    # them: rint then decides every code, so any quotient off by one ulp
    # changes one.
    rng = np.random.default_rng(1420)
    K, N = 1024, 16
    exps = [-130, -126, -125, -101, -100, -99, -20, -1, 0, 1, 20, 100, 120]
    rows = []
    for e in exps:
        for _ in range(4):
            a = np.float32(np.ldexp(rng.uniform(1.0, 2.0), e) * 127.0)
            sx = np.float32(a / np.float32(127.0))
            k = rng.integers(-127, 127, size=K).astype(np.float32)
            x = (sx * (k + np.float32(0.5))).astype(np.float32)
            sel = rng.integers(0, 3, size=K)
            x = np.where(sel == 1, np.nextafter(x, np.float32(np.inf)), x)
            x = np.where(sel == 2, np.nextafter(x, np.float32(-np.inf)), x)
            x = np.clip(x, -a, a).astype(np.float32)
            x[0] = a                                  # the row's maximum
            rows.append(x)
    X = np.stack(rows).astype(np.float32)
    Wq = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    Sw = np.ones(N, np.float32)
    _, Xq, Sx, _ = wq.gemm_w8a8(cu(X), cu(Wq), cu(Sw), want_acc=True)
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):  # Y overflows at the largest scales; only Xq, Sx are checked
        r = oracle.gemm_w8a8(X, Wq, Sw)
    assert np.array_equal(Sx.cpu().numpy().view(np.uint32), r["Sx"].view(np.uint32))
    got = Xq.cpu().numpy()
    bad = np.nonzero((got != r["Xq"]).any(axis=1))[0]
    assert bad.size == 0, (
        f"rows {bad.tolist()} (scale exponents {[exps[i // 4] for i in bad]}): "
        f"{int((got != r['Xq']).sum())} codes differ, max |diff| "
        f"{int(np.abs(got.astype(np.int32) - r['Xq'].astype(np.int32)).max())}")


# ----------------------------------------------------- SmoothQuant (W8A8) --

@pytest.mark.parametrize("M,K,N", [(32, 1024, 64), (130, 256, 528), (7, 12288, 96),
                                   (256, 8192, 8192)])
def test_w8a8_smooth_bit_exact(wq, M, K, N):
    # Outlier activation channels; the quantiser divides X by s, the GEMM is
    # the plain W8A8 one on diag(s) W.  Codes, scales, accumulators and bf16
    # output bits all equal the oracle's.  K = 12288 takes the quantiser's
    # two-pass path (rows longer than one register block).
    d = synth.gen_w8a8_smooth(M, K, N, seed=synth.SEEDS["w8a8_smooth"] + M + K + N)
    Y, Xq, Sx, acc = wq.gemm_w8a8(cu(d["X"]), cu(d["Wq"]), cu(d["Sw"]), want_acc=True,
                                  smooth=cu(d["smooth"]))
    torch.cuda.synchronize()
    r = oracle.gemm_w8a8_smooth(d["X"], d["smooth"], d["Wq"], d["Sw"])
    assert np.array_equal(Xq.cpu().numpy(), r["Xq"])
    assert np.array_equal(Sx.cpu().numpy().view(np.uint32), r["Sx"].view(np.uint32))
    assert np.array_equal(acc.cpu().numpy(), r["acc"])
    assert np.array_equal(Y.view(torch.int16).cpu().numpy().view(np.uint16), r["y_bits"])


def test_w8a8_smooth_ones_equals_plain(wq):
    d = synth.gen_w8a8(64, 640, 64, seed=73)
    X, Wq, Sw = cu(d["X"]), cu(d["Wq"]), cu(d["Sw"])
    a = wq.gemm_w8a8(X, Wq, Sw, want_acc=True, smooth=torch.ones(640, dtype=torch.float32, device=dev()))
    b = wq.gemm_w8a8(X, Wq, Sw, want_acc=True)
    for t1, t2 in zip(a, b):
        assert torch.equal(t1, t2)


# ------------------------------------------------ LLM.int8() decomposition --

def _mixed_check(wq, X16, W16, threshold):
    Y, Xq, Sx, Wq, Sw, colmax, mask, cols, n_out, acc = wq.gemm_int8_mixed(cu(X16), cu(W16), threshold,
                                                                           want_acc=True)
    torch.cuda.synchronize()
    r = oracle.int8_mixed_decompose(X16, W16, threshold)
    K = X16.shape[1]
    assert np.array_equal(colmax.cpu().numpy().view(np.uint32), r["colmax"].view(np.uint32))
    bits = np.zeros(K, np.uint8)
    bits[r["cols"]] = 1
    assert np.array_equal(mask.cpu().numpy().view(np.uint32),
                          np.packbits(bits, bitorder="little").view("<u4"))
    assert int(n_out.item()) == r["cols"].size
    assert np.array_equal(cols.cpu().numpy()[:r["cols"].size], r["cols"])
    assert np.array_equal(Xq.cpu().numpy(), r["Xq"])
    assert np.array_equal(Sx.cpu().numpy().view(np.uint32), r["Sx"].view(np.uint32))
    assert np.array_equal(Wq.cpu().numpy(), r["Wq"])
    assert np.array_equal(Sw.cpu().numpy().view(np.uint32), r["Sw"].view(np.uint32))
    assert np.array_equal(acc.cpu().numpy(), r["acc"])
    y = host(Y)
    what = f"int8 mixed {X16.shape[0]}x{K}x{W16.shape[0]} thr {threshold}"
    if np.any(r["y_exact"]):
        assert_tol(y, r["y_exact"], what)
    # the int8 part reaches fp32 through three roundings (float(acc), * Sx,
    # * Sw); the fp16 part sums exact products of the outlier columns
    c = r["cols"]
    abs_sum = np.abs(r["y_int8"]) + np.abs(X16[:, c].astype(np.float64)) @ np.abs(W16[:, c].astype(np.float64)).T
    assert_fwd_bound(y, r["y_exact"], abs_sum, c.size + 3, "f16", what)
    return r


@pytest.mark.parametrize("M,K,N,nout", [(32, 1024, 64, 8), (130, 256, 528, 3), (7, 2048, 96, 0),
                                        (256, 8192, 8192, 8)])
def test_int8_mixed_vs_oracle(wq, M, K, N, nout):
    # Outlier channels 20x (beyond 6.0): the scan, the outlier list, the
    # quantised regular part of X and W and the int32 accumulators equal the
    # oracle's bit for bit; the fp16 output meets the tolerance and the
    # forward error bound against the exact sum of the two parts.
    d = synth.gen_int8_mixed(M, K, N, seed=synth.SEEDS["int8_mixed"] + M + K + N, n_outlier=nout)
    r = _mixed_check(wq, d["X"], d["W16"], 6.0)
    assert np.array_equal(r["cols"], d["outlier_cols"])


def test_int8_mixed_worked_example(wq):
    # The hand-worked example of tests/golden/int8_mixed_worked.txt, padded
    # with zero columns (K = 64) and zero output channels (N = 16); every
    # step is exact in fp32, so Y is the fp16 rounding of the fixture's y.
    from conftest import read_golden
    rows = {k: v for k, v in read_golden("int8_mixed_worked.txt")}
    f = lambda key: np.array([float(t) for t in rows[key].split()])
    X = np.zeros((2, 64), np.float16)
    W = np.zeros((16, 64), np.float16)
    X[:, :4] = f("X").reshape(2, 4)
    W[:2, :4] = f("W").reshape(2, 4)
    Y, Xq, Sx, Wq, Sw, colmax, mask, cols, n_out, acc = wq.gemm_int8_mixed(cu(X), cu(W), 6.0, want_acc=True)
    torch.cuda.synchronize()
    assert int(n_out.item()) == 1 and int(cols[0].item()) == 2
    assert Xq.cpu().numpy()[:, :4].ravel().tolist() == f("Xq").astype(int).tolist()
    assert Wq.cpu().numpy()[:2, :4].ravel().tolist() == f("Wq").astype(int).tolist()
    assert Sx.cpu().numpy().tolist() == f("Sx").tolist()
    assert Sw.cpu().numpy()[:2].tolist() == f("Sw").tolist()
    assert acc.cpu().numpy()[:, :2].ravel().tolist() == f("acc").astype(int).tolist()
    y = host(Y)
    assert y[:, :2].ravel().tolist() == f("y").astype(np.float16).astype(np.float64).tolist()
    assert np.all(y[:, 2:] == 0)


def test_int8_mixed_thresholds_and_zero_rows(wq):
    rng = np.random.default_rng(83)
    M, K, N = 5, 128, 32
    X = rng.standard_normal((M, K)).astype(np.float16)
    X[:, 7] = 40.0                       # an outlier column
    X[3, :] = 0
    X[3, 7] = 9.0                        # row 3: only its outlier value is non-zero
    W = rng.normal(0, 0.02, size=(N, K)).astype(np.float16)
    W[4, :] = 0
    W[4, 7] = 0.5                        # channel 4: only its outlier entry is non-zero
    r = _mixed_check(wq, X, W, 6.0)
    assert r["cols"].tolist() == [7] and r["Sx"][3] == 0 and r["Sw"][4] == 0
    _mixed_check(wq, X, W, 1e30)    # nothing taken out
    _mixed_check(wq, X, W, -1.0)    # every column taken out


# ====================================================== large activations ==

def _with_large_entries(x, rows, value=60000.0):
    x = np.array(x, copy=True)
    for i, k in enumerate(rows):
        x[..., k] = value if i % 2 == 0 else -value
    return x


def test_large_fp16_activations_all_paths(wq):
    """fp16 activations near the top of the fp16 range (60000) at a few rows,
    the rest N(0,1): every weight-only path stays finite and within the
    tolerance (outputs stay inside the fp16 range)."""
    rows = (3, 100, 517, 1000)
    d = synth.gen_q3(1024, 256, seed=81, dtype="f16")
    x = _with_large_entries(d["x"], rows).astype(np.float16)
    y = wq.matvec_q3(cu(x), wq.prepack_q3(cu(d["qweight"]), 1024), cu(d["scales"]), cu(d["zeros"]))
    assert_tol(host(y), oracle.matvec_q3(x, d["qweight"], d["scales"], d["zeros"]), "q3 f16 large x")

    d = synth.gen_q8_group(2, 1024, 256, 128, seed=82)
    X = _with_large_entries(d["X"], rows).astype(np.float16)
    y = wq.gemm_q8_group(cu(X), wq.prepack_q8(cu(d["q"])), cu(d["scales"]), 128)
    assert_tol(host(y), oracle.gemm_q8_group(X, d["q"], d["scales"], 128), "q8 large x")

    d = synth.gen_q4_group(2, 1024, 256, 128, seed=83, act_order=True)
    X = _with_large_entries(d["X"], rows).astype(np.float16)
    packed, _ = wq.prepare_q4(cu(d["qweight"]), d["g_idx"], 128)
    y = wq.gemm_q4_group(cu(X), packed, cu(d["scales"]), 128)
    assert_tol(host(y), oracle.gemm_q4_group(X, d["qweight"], d["scales"], d["g_idx"], 128), "q4 large x")

    d = synth.gen_q2_zp(2, 1024, 256, 128, seed=84, act_order=True)
    X = _with_large_entries(d["X"], rows).astype(np.float16)
    packed, _ = wq.prepare_q2(cu(d["qweight"]), d["g_idx"], 128)
    y = wq.gemm_q2_group_zp(cu(X), packed, cu(d["scales"]), cu(d["zeros"]), 128)
    assert_tol(host(y), oracle.gemm_q2_zp(X, d["qweight"], d["scales"], d["zeros"], d["g_idx"], 128),
               "q2 large x")


def test_large_fp32_activations_q3(wq):
    """fp32 3-bit matvec with |x| far beyond any fp16 range: a few rows at
    +-2^110 over N(0,1), then every row scaled by 2^100.  The products stay
    finite in fp32 (|y| ~ 2^110), so the kernel must too: no step may scale
    x up on its way in."""
    d = synth.gen_q3(1024, 256, seed=85, dtype="f32")
    packed = wq.prepack_q3(cu(d["qweight"]), 1024)
    for x in (_with_large_entries(d["x"], (3, 100, 517, 1000), value=2.0 ** 110).astype(np.float32),
              (d["x"].astype(np.float64) * 2.0 ** 100).astype(np.float32)):
        y = host(wq.matvec_q3(cu(x), packed, cu(d["scales"]), cu(d["zeros"])))
        assert np.isfinite(y).all()
        assert_tol(y, oracle.matvec_q3(x, d["qweight"], d["scales"], d["zeros"]), "q3 f32 large x")


# ============================================================ measurement ==

@pytest.mark.parametrize("nbytes,pos", [(1 << 24, 0), (1 << 24, (1 << 24) - 4), (65536 * 3 + 48, 65536 * 3 + 36),
                                        (4096, 2052)])
def test_calib_stream_reads_every_byte(wq, nbytes, pos):
    """The bare-stream reference reads each word of the buffer: a single
    non-zero word equal to the sink's trigger value, anywhere (ragged tails
    included), is seen by exactly the thread whose loads cover it."""
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev())
    sink = torch.zeros(1, dtype=torch.int32, device=dev())
    wq.calib_stream_read(buf, sink)
    wq.calib_empty(sink, 256, 512)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    buf[pos // 4] = np.int32(np.uint32(0x9E3779B9).view(np.int32))
    wq.calib_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == 0x9E3779B9
