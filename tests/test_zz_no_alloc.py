"""The no-allocation W8A8 entry point against wq_gemm_w8a8 (GPU, through the C ABI).

wq_gemm_w8a8_noalloc takes its split-K workspace from the library's own
device array instead of a caller buffer.  Its outputs must equal those of
wq_gemm_w8a8 bit for bit (Xq, the Sx bits, the int32 accumulators and the
bf16 output), on two calls in a row, the second smaller, so that whatever
the first call left in the array does not leak into the second.
"""
import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _cu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda:0"))


def test_noalloc_matches_w8a8_on_two_calls():
    import weight_only_quantized_dequant_amd as wq
    wq.lib()
    for M, K, N, seed in ((256, 8192, 8192, 1400), (64, 2048, 1024, 91)):
        print(f"no-alloc W8A8 M={M} K={K} N={N}", flush=True)
        d = synth.gen_w8a8(M, K, N, seed=seed)
        X, Wq, Sw = _cu(d["X"]), _cu(d["Wq"]), _cu(d["Sw"])
        Y0, Xq0, Sx0, acc0 = wq.gemm_w8a8(X, Wq, Sw, want_acc=True)
        dev = X.device
        Y = torch.full((M, N), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
        Xq = torch.full((M, K), 55, dtype=torch.int8, device=dev)
        Sx = torch.full((M,), -3.0, dtype=torch.float32, device=dev)
        acc = torch.full((M, N), 123456, dtype=torch.int32, device=dev)
        wq.gemm_w8a8_noalloc(X, Wq, Sw, Y, Xq, Sx, acc)
        torch.cuda.synchronize()
        assert torch.equal(Xq, Xq0)
        assert torch.equal(Sx.view(torch.int32), Sx0.view(torch.int32))
        assert torch.equal(acc, acc0)
        assert torch.equal(Y.view(torch.int16), Y0.view(torch.int16))


def test_noalloc_rejects_a_shape_beyond_its_array():
    import weight_only_quantized_dequant_amd as wq
    M, K, N = 256, 8192, 8704        # two K slices of 256 x 8704 int32: 17 MiB > 16 MiB
    assert wq.workspace_bytes(wq.WQ_OP_W8A8, M, K, N) > (16 << 20)
    dev = torch.device("cuda:0")
    X = torch.zeros((M, K), dtype=torch.float32, device=dev)
    Wq = torch.zeros((N, K), dtype=torch.int8, device=dev)
    Sw = torch.zeros(N, dtype=torch.float32, device=dev)
    Y = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
    Xq = torch.zeros((M, K), dtype=torch.int8, device=dev)
    Sx = torch.zeros(M, dtype=torch.float32, device=dev)
    with pytest.raises(wq.WQError) as e:
        wq.gemm_w8a8_noalloc(X, Wq, Sw, Y, Xq, Sx)
    assert e.value.status == wq.WQ_ERR_WORKSPACE
