"""Host-side logic that needs no GPU: the benchmark's contract and byte
counts, and the binding's refusal to compute anywhere but on the device."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
torch = pytest.importorskip("torch")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_bench_algorithmic_bytes():
    sys.path.insert(0, ROOT)
    import bench
    import weight_only_quantized_dequant_amd as wq
    dev = torch.device("cpu")  # nothing is placed on it: the byte counts need no device
    # int8 GEMV, M = 1, K = N = 4096, group 128: codes + fp32 scales + x + y
    assert bench.wl_q8(wq, torch, dev).nbytes == 4096 * 4096 + 32 * 4096 * 4 + 4096 * 2 + 4096 * 2 == 17317888
    # 4-bit act-order, M = 1, K = 4096, N = 11008: codes + fp16 scales + uint16 row table + x + y
    assert bench.wl_q4(wq, torch, dev, 1).nbytes == 4096 * 11008 // 2 + 32 * 11008 * 2 + 4096 * 2 + 4096 * 2 + 11008 * 2
    # 3-bit fp16, K = N = 4096: 3 bits per code + scale and zero per column + x + y
    assert bench.wl_q3(wq, torch, dev, 4096, 4096, "f16", 1200).nbytes == 4096 * 4096 * 3 // 8 + 4 * 4096 + 2 * 4096 + 2 * 4096
    # 2-bit asymmetric, M = 1, K = 4096, N = 11008, group 128: codes + fp16 scales and zeros
    # + uint16 row table + x + y
    assert bench.wl_q2(wq, torch, dev, 1).nbytes == (4096 * 11008 // 4 + 2 * 32 * 11008 * 2 + 4096 * 2
                                                     + 4096 * 2 + 11008 * 2) == 12719616
    assert bench._rotation(17317888) == 32      # >= 512 MB of rotated copies


def test_binding_refuses_host_tensors():
    # No CPU fallback: the product path takes device tensors only.
    import synth
    import weight_only_quantized_dequant_amd as wq
    d = synth.gen_q8_group(1, 256, 16, 128, seed=5)
    with pytest.raises(ValueError, match="device tensor"):
        wq.gemm_q8_group(torch.from_numpy(d["X"]), torch.zeros(256 * 16, dtype=torch.uint8),
                         torch.from_numpy(d["scales"]), 128)
    d = synth.gen_w8a8(4, 64, 16, seed=6)
    with pytest.raises(ValueError, match="device tensor"):
        wq.gemm_w8a8(torch.from_numpy(d["X"]), torch.from_numpy(d["Wq"]), torch.from_numpy(d["Sw"]))


def test_oracle_is_not_imported_by_the_product():
    # The product package never imports the oracle (only tests, smoke and the
    # benchmark's CPU-baseline leg may).
    pkg = os.path.join(ROOT, "weight_only_quantized_dequant_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h", ".hpp")):
                with open(os.path.join(dirpath, f), encoding="utf-8") as fh:
                    text = fh.read()
                assert "import oracle" not in text and "from oracle" not in text, f
