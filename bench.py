"""Benchmark of the fused dequantize-and-multiply kernels on one MI355X.

Default workload: the M=1 group-wise int8 weight-only GEMV, K = N = 4096,
group 128 (fp16 activations, fp32 accumulation, fp16 output).  One step is
one call of the fused kernel on one batch of synthetic input.  The metric is
achieved HBM bandwidth over the algorithmic bytes of a call (packed weight,
scales and activations read once, output written once), as GB/s and as a
fraction of the 8 TB/s HBM3E peak.

Inputs sit in HBM before timing starts.  To keep the weights from being
served by the 256 MB Infinity Cache or the L2s, the argument set is
replicated R times (R * bytes >= 512 MB) and the steps cycle through the
copies.  Time is taken with HIP events on the stream the kernels are
launched on, bracketing exactly `--steps` calls after `--warmup` untimed
ones.  Before each timed region a pre-roll of one call per copy evicts the
copies the timed calls read, and a spin kernel keeps the GPU busy until all
timed calls are queued, so the events see the kernels back to back.  The
timed region is repeated (--trials) and the median is reported.

Extra fields on the single JSON line:
* roofline: the dominant (only) kernel's bandwidth against 8 TB/s; "traffic"
  comes from the rocprofv3 counter summary committed under profiles/ when it
  was taken on the current kernel source, else null.
* cpu_baseline: the CPU oracle (numpy, fp64) timed on this host on the same
  workload, in child processes started before the GPU is touched: one leg
  with the job's BLAS thread count and one with a single thread, each about
  8 s of calls timed one by one (median), with the host's visible cores and
  CPU model.
* calibration (headline only): an empty kernel with the GEMV's grid (the
  dispatch floor) and a kernel that only streams each copy's packed weight
  once with the GEMV's loads (the achievable time for those bytes here), on
  the same rotation and graph replay.
* secondary (unless --headline-only): the other workloads of the library,
  each as microseconds per call and GB/s (or TOPS) with the same method, and
  (unless --no-calibration) the time of a bare stream of the same weight
  bytes on the same rotation, with the kernel's share of it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0     # dense int8 MFMA, POP/s x 1e-12
FP16_PEAK_TFLOPS = 2500.0   # dense fp16 MFMA
FP32_PEAK_TFLOPS = 157.3    # dense fp32 MFMA
MALL_BYTES = 256 << 20


def _sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "q8_group": ["weight_only_quantized_dequant_amd/csrc/q8_group.hip",
                 "weight_only_quantized_dequant_amd/csrc/wq_device.hpp"],
}


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if current."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha") != _sha(KERNEL_SOURCES[kernel]):
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------- workloads --

class Workload:
    """One configuration: builds R device copies and runs one step on copy i."""

    def __init__(self, name, nbytes, make, run, flops=0):
        self.name, self.nbytes, self.make, self.run, self.flops = name, nbytes, make, run, flops


def _rotation(nbytes, floor=2 * MALL_BYTES, cap=64):
    return int(min(cap, max(1, -(-floor // nbytes))))


def wl_q8(wq, torch, dev, M=1):
    import synth
    K, N, G = 4096, 4096, 128
    nbytes = K * N + (K // G) * N * 4 + M * K * 2 + M * N * 2
    d = synth.gen_q8_group(M, K, N, G, seed=synth.SEEDS["q8_group_4096" if M == 1 else "q8_group_m512"])

    def make(R):
        base = [torch.from_numpy(d["X"]).to(dev), wq.prepack_q8(torch.from_numpy(d["q"]).to(dev)),
                torch.from_numpy(d["scales"]).to(dev)]
        # one workspace (the K slices' partial tiles, above 32 rows) serves every copy
        nws = wq.workspace_bytes(wq.WQ_OP_Q8G, M, K, N)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        copies = [[t.clone() for t in base] + [torch.empty((M, N), dtype=torch.float16, device=dev), ws]
                  for _ in range(R)]
        return copies

    def run(c):
        wq.gemm_q8_group(c[0], c[1], c[2], G, Y=c[3], ws=c[4])

    kind = "gemv" if M == 1 else "streaming" if M <= 32 else "gemm"
    w = Workload(f"q8_group_{kind} M={M} K={K} N={N} G={G}", nbytes, make, run,
                 flops=0 if M == 1 else 2 * M * K * N)
    w.peak_tops = FP16_PEAK_TFLOPS
    w.config = {"workload": w.name, "M": M, "K": K, "N": N, "group": G}
    w.oracle = lambda: __import__("oracle").gemm_q8_group(d["X"], d["q"], d["scales"], G)
    w.dtype = "int8 weight x fp16 act, fp32 accumulate"
    return w


def wl_q3(wq, torch, dev, K, N, dt, seed):
    import synth
    esz = 4 if dt == "f32" else 2
    nbytes = (K // 32) * 3 * N * 4 + 2 * N * esz + K * esz + N * esz
    d = synth.gen_q3(K, N, seed=seed, dtype=dt)

    def make(R):
        base = [torch.from_numpy(a).to(dev) for a in (d["x"], d["qweight"], d["scales"], d["zeros"])]
        base[1] = wq.prepack_q3(base[1], K)
        return [[t.clone() for t in base] + [torch.empty(N, dtype=base[0].dtype, device=dev)]
                for _ in range(R)]

    def run(c):
        wq.matvec_q3(c[0], c[1], c[2], c[3], y=c[4])

    w = Workload(f"q3_matvec_{dt} K={K} N={N}", nbytes, make, run)
    w.oracle = lambda: __import__("oracle").matvec_q3(d["x"], d["qweight"], d["scales"], d["zeros"])
    return w


def wl_q4(wq, torch, dev, M):
    import synth
    K, N, G = 4096, 11008, 128
    # packed codes + scales + the uint16 row table + X + Y
    nbytes = (K // 8) * N * 4 + (K // G) * N * 2 + K * 2 + M * K * 2 + M * N * 2
    d = synth.gen_q4_group(M, K, N, G, seed=synth.SEEDS["q4_group_actorder"])

    def make(R):
        qw = torch.from_numpy(d["qweight"]).to(dev)
        packed, _ = wq.prepare_q4(qw, d["g_idx"], G)
        base = [torch.from_numpy(d["X"]).to(dev), packed, torch.from_numpy(d["scales"]).to(dev)]
        # one workspace (X in the packed row order, above 4 rows) serves every copy
        nws = wq.workspace_bytes(wq.WQ_OP_Q4G, M, K, N)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        return [[t.clone() for t in base] + [torch.empty((M, N), dtype=torch.float16, device=dev), ws]
                for _ in range(R)]

    def run(c):
        wq.gemm_q4_group(c[0], c[1], c[2], G, Y=c[3], ws=c[4])

    w = Workload(f"q4_group_actorder M={M} K={K} N={N} G={G}", nbytes, make, run)
    w.oracle = lambda: __import__("oracle").gemm_q4_group(d["X"], d["qweight"], d["scales"], d["g_idx"], G)
    return w


def wl_int8_mixed(wq, torch, dev):
    import synth
    M, K, N = 256, 8192, 8192
    # column scan: read X fp16, write colmax + mask; quantiser: read X and W
    # fp16 (and the mask), write Xq, Sx, Wq, Sw; GEMM: read Xq, Wq, Sx, Sw,
    # write Y fp16 (the outlier columns of X and W are a few KB)
    nbytes = ((2 * M * K + 4 * K + K // 8) + (2 * M * K + 2 * N * K + M * K + 4 * M + N * K + 4 * N)
              + (M * K + N * K + 4 * M + 4 * N + 2 * M * N))
    d = synth.gen_int8_mixed(M, K, N, seed=synth.SEEDS["int8_mixed"])

    def make(R):
        base = [torch.from_numpy(a).to(dev) for a in (d["X"], d["W16"])]
        ws = torch.empty(max(16, wq.workspace_bytes(wq.WQ_OP_W8A8, M, K, N)), dtype=torch.uint8, device=dev)
        return [[t.clone() for t in base] + [torch.empty((M, N), dtype=torch.float16, device=dev), ws]
                for _ in range(R)]

    def run(c):
        wq.gemm_int8_mixed(c[0], c[1], 6.0, Y=c[2], ws=c[3])

    w = Workload(f"int8_mixed_decomposition M={M} K={K} N={N} outlier_cols=8", nbytes, make, run,
                 flops=2 * M * K * N)
    w.peak_tops = INT8_PEAK_TOPS
    w.oracle = lambda: __import__("oracle").int8_mixed_decompose(d["X"], d["W16"], 6.0)
    return w


def wl_q4zp(wq, torch, dev, M, G=128, act=False):
    import synth
    K, N = 4096, 11008
    # packed codes + scales + zeros + the uint16 row table + X + Y
    nbytes = (K // 8) * N * 4 + 2 * (K // G) * N * 2 + K * 2 + M * K * 2 + M * N * 2
    d = synth.gen_q4_zp(M, K, N, G, seed=synth.SEEDS["q4_zp"], act_order=act)

    def make(R):
        packed, _ = wq.prepare_q4(torch.from_numpy(d["qweight"]).to(dev), d["g_idx"] if act else None, G)
        base = [torch.from_numpy(d["X"]).to(dev), packed, torch.from_numpy(d["scales"]).to(dev),
                torch.from_numpy(d["zeros"]).to(dev)]
        nws = wq.workspace_bytes(wq.WQ_OP_Q4G, M, K, N)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        return [[t.clone() for t in base] + [torch.empty((M, N), dtype=torch.float16, device=dev), ws]
                for _ in range(R)]

    def run(c):
        wq.gemm_q4_group_zp(c[0], c[1], c[2], c[3], G, Y=c[4], ws=c[5])

    w = Workload(f"q4_zp_asymmetric{' act-order' if act else ''} M={M} K={K} N={N} G={G}", nbytes, make, run)
    w.oracle = lambda: __import__("oracle").gemm_q4_zp(d["X"], d["qweight"], d["scales"], d["zeros"],
                                                       d["g_idx"] if act else None, G)
    return w


def wl_q2(wq, torch, dev, M, G=128):
    import synth
    K, N = 4096, 11008
    # packed codes + scales + zeros + the uint16 row table + X + Y
    nbytes = (K // 16) * N * 4 + 2 * (K // G) * N * 2 + K * 2 + M * K * 2 + M * N * 2
    d = synth.gen_q2_zp(M, K, N, G, seed=synth.SEEDS["q2_zp"])

    def make(R):
        packed, _ = wq.prepare_q2(torch.from_numpy(d["qweight"]).to(dev), None, G)
        base = [torch.from_numpy(d["X"]).to(dev), packed, torch.from_numpy(d["scales"]).to(dev),
                torch.from_numpy(d["zeros"]).to(dev)]
        return [[t.clone() for t in base] + [torch.empty((M, N), dtype=torch.float16, device=dev)]
                for _ in range(R)]

    def run(c):
        wq.gemm_q2_group_zp(c[0], c[1], c[2], c[3], G, Y=c[4])

    w = Workload(f"q2_zp_asymmetric M={M} K={K} N={N} G={G}", nbytes, make, run)
    w.oracle = lambda: __import__("oracle").gemm_q2_zp(d["X"], d["qweight"], d["scales"], d["zeros"], None, G)
    return w


def wl_q8_separated(wq, torch, dev, M=512, dt="f16"):
    """The unfused comparator of the fused int8 product at the fused-kernel
    page's workload: the dequantisation kernel writes the whole fp16 (or fp32)
    weight, then a library GEMM (torch.matmul) reads it."""
    import synth
    K, N, G = 4096, 4096, 128
    b = 2 if dt == "f16" else 4
    # dequant: read codes + scales, write W; GEMM: read X and W, write Y
    nbytes = (K * N + (K // G) * N * 4 + K * N * b) + (M * K * b + K * N * b + M * N * b)
    d = synth.gen_q8_group(M, K, N, G, seed=synth.SEEDS["q8_group_m512"])
    tdt = torch.float16 if dt == "f16" else torch.float32

    def make(R):
        X = torch.from_numpy(d["X"]).to(dev).to(tdt)
        base = [X, torch.from_numpy(d["q"]).to(dev), torch.from_numpy(d["scales"]).to(dev)]
        W = torch.empty((K, N), dtype=tdt, device=dev)   # the intermediate every call rewrites
        return [[t.clone() for t in base] + [W, torch.empty((M, N), dtype=tdt, device=dev)]
                for _ in range(R)]

    def run(c):
        wq.dequant_q8_group(c[1], c[2], G, tdt, W=c[3])
        torch.matmul(c[0], c[3], out=c[4])

    w = Workload(f"q8_group_separated_{dt} M={M} K={K} N={N} G={G}", nbytes, make, run,
                 flops=2 * M * K * N)
    w.peak_tops = FP16_PEAK_TFLOPS if dt == "f16" else FP32_PEAK_TFLOPS
    w.config = {"workload": w.name, "M": M, "K": K, "N": N, "group": G,
                "form": f"dequant kernel writes {dt} W, then torch.matmul"}
    w.oracle = lambda: __import__("oracle").gemm_q8_group(d["X"], d["q"], d["scales"], G)
    w.dtype = f"{dt} weight x {dt} act, library GEMM"
    return w


def wl_w8a8(wq, torch, dev, smooth=False, resident=False):
    import synth
    M, K, N = 256, 8192, 8192
    # quantiser: read X fp32 (and s), write Xq + Sx; GEMM: read Xq, Wq, Sx, Sw, write Y.
    # The split-K partials (S * M * N int32, written and read back once) are
    # the kernel's own traffic, not the method's: they are not counted.
    nbytes = (M * K * 4 + M * K + M * 4) + (M * K + N * K + M * 4 + N * 4 + M * N * 2)
    if smooth:
        nbytes += K * 4
        d = synth.gen_w8a8_smooth(M, K, N, seed=synth.SEEDS["w8a8_smooth"])
    else:
        d = synth.gen_w8a8(M, K, N, seed=synth.SEEDS["w8a8_256x8192x8192"])

    def make(R):
        base = [torch.from_numpy(a).to(dev) for a in (d["X"], d["Wq"], d["Sw"])]
        extra = [torch.from_numpy(d["smooth"]).to(dev)] if smooth else [None]
        # one workspace serves every copy: the calls run one after another
        ws = torch.empty(max(16, wq.workspace_bytes(wq.WQ_OP_W8A8, M, K, N)), dtype=torch.uint8, device=dev)
        return [[t.clone() for t in base] + [torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                                             torch.empty((M, K), dtype=torch.int8, device=dev),
                                             torch.empty(M, dtype=torch.float32, device=dev)]
                + [t.clone() if t is not None else None for t in extra] + [ws]
                for _ in range(R)]

    def run(c):
        wq.gemm_w8a8(c[0], c[1], c[2], Y=c[3], Xq=c[4], Sx=c[5], smooth=c[6], ws=c[7])

    kind = "w8a8_smoothquant" if smooth else "w8a8_dynamic"
    name = f"{kind} M={M} K={K} N={N}"
    if resident:
        # One argument set, every call: the 67 MB of Wq stay in the 256 MB
        # Infinity Cache, so the line shows the matrix-core side of the call,
        # not HBM.  Reported apart from the HBM-resident line.
        name += " (cache-resident: one argument set)"
    w = Workload(name, nbytes, make, run, flops=2 * M * K * N)
    if resident:
        w.rotation = 1
    w.peak_tops = INT8_PEAK_TOPS
    w.oracle = lambda: __import__("oracle").gemm_w8a8(d["X"], d["Wq"], d["Sw"])
    return w


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


_SPIN_CYCLES_PER_MS = None


def _spin_rate(torch):
    """Cycles per millisecond of torch's spin kernel on this GPU (measured once)."""
    global _SPIN_CYCLES_PER_MS
    if _SPIN_CYCLES_PER_MS is None:
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(2_000_000)
        b.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS = 2_000_000 / a.elapsed_time(b)
    return _SPIN_CYCLES_PER_MS


def time_workload(torch, w, steps, warmup, R=None, trials=None, method="eager"):
    """Time of one step: the median over trials of exactly `steps` back-to-back steps.

    Every trial, on the current stream (the one the library launches on):
    1. a pre-roll, one call on each of the R copies, replayed from a captured
       graph: when timed call i runs, the R - 1 other copies (>= 512 MB for
       the streaming workloads) have been read since copy i was, so its
       weights come from HBM, not from the 256 MB Infinity Cache or the L2s;
    2. a spin kernel that holds the GPU for twice the host time of issuing
       `steps` calls (measured on an untimed pass), so the timed calls are
       all queued before the first one starts;
    3. the start event, exactly `steps` calls (call i on copy i mod R) issued
       one by one through the library, the end event.
    The step time is the events' elapsed time over `steps`; the median over
    trials is returned.  method="graph" instead replays a captured graph of
    the `steps` calls between the events (each replay then adds a fixed
    cost of several microseconds on the GPU).
    Returns (median ms per step, R, per-trial ms per step).
    """
    R = R or getattr(w, "rotation", None) or _rotation(w.nbytes)
    copies = w.make(R)
    for i in range(warmup):
        w.run(copies[i % R])
    torch.cuda.synchronize()
    if trials is None:
        trials = 11 if steps <= 500 else 5
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    preroll, timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        w.run(copies[0])  # first call on the side stream, outside the capture
        torch.cuda.current_stream().synchronize()
        with torch.cuda.graph(preroll, stream=side):
            for i in range(R):
                w.run(copies[i])
        if method == "graph":
            with torch.cuda.graph(timed, stream=side):
                for i in range(steps):
                    w.run(copies[i % R])
    torch.cuda.synchronize()
    preroll.replay()  # untimed: the first replay of a graph uploads it
    if method == "graph":
        timed.replay()
    t0 = time.perf_counter()
    for i in range(steps):
        w.run(copies[i % R])
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    spin = int(_spin_rate(torch) * (2.0 * host_ms + 0.2))
    per = []
    for _ in range(trials):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        preroll.replay()
        torch.cuda._sleep(spin)
        start.record()
        if method == "graph":
            timed.replay()
        else:
            for i in range(steps):
                w.run(copies[i % R])
        end.record()
        torch.cuda.synchronize()
        per.append(start.elapsed_time(end) / steps)
    del preroll, timed, copies
    torch.cuda.empty_cache()
    return _median(per), R, per


def calibration(wq, torch, w, steps, warmup, gemv_ms):
    """Dispatch floor and achievable streaming time for the headline workload.

    Same rotation and graph replay as the GEMV: (a) an empty kernel with the
    GEMV's grid (256 x 512 threads), (b) a kernel that only reads each copy's
    packed weight once with the GEMV's loads.  The GEMV moves the same weight
    plus 2.6% more bytes, so (b) is a lower bound for it on this GPU.
    """
    dev = torch.device("cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def run_stream(c):
        wq.calib_stream_read(c[1], sink)

    sw = Workload("stream read of the packed weight", w.nbytes, w.make, run_stream)
    s_ms, R, _ = time_workload(torch, sw, steps, warmup)
    ew = Workload("empty kernel", 0, lambda R: [[None]] * R, lambda c: wq.calib_empty(sink, 256, 512))
    e_ms, _, _ = time_workload(torch, ew, steps, warmup, R=1)
    wbytes = w.make(1)[0][1].numel()
    return {"empty_kernel_us": round(e_ms * 1e3, 3), "stream_read_us": round(s_ms * 1e3, 3),
            "stream_read_bytes": wbytes, "stream_read_GB_per_s": round(wbytes / (s_ms * 1e-3) / 1e9, 1),
            "stream_read_pct_hbm_peak": round(100 * wbytes / (s_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "share_of_stream_ceiling": round(s_ms / gemv_ms, 4), "rotation_copies": R}


def stream_sweep(wq, torch, dev, steps, warmup):
    """The per-launch streaming ceiling: a kernel that only reads `size` bytes
    with the int8 GEMV's loads (wq_calib_stream_read), at 4..256 MiB, timed
    like every workload (rotated copies, queued launches, median of trials);
    and the empty kernel with the GEMV's grid (the dispatch floor)."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ew = Workload("empty kernel", 0, lambda R: [[None]] * R, lambda c: wq.calib_empty(sink, 256, 512))
    e_ms, _, _ = time_workload(torch, ew, steps, warmup, R=1)
    print(json.dumps({"kernel": "calib_empty", "grid": 256, "threads": 512,
                      "us": round(e_ms * 1e3, 3)}), flush=True)
    for mib in (4, 8, 16, 32, 64, 128, 256):
        nbytes = mib << 20
        sw = Workload(f"stream {mib} MiB", nbytes,
                      lambda R, n=nbytes: [[torch.empty(n // 4, dtype=torch.int32, device=dev).fill_(1)]
                                           for _ in range(R)],
                      lambda c: wq.calib_stream_read(c[0], sink))
        ms, R, _ = time_workload(torch, sw, steps, warmup)
        print(json.dumps({"kernel": "calib_stream_read", "MiB": mib, "bytes": nbytes, "rotation_copies": R,
                          "us": round(ms * 1e3, 3), "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}),
              flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(name, budget_s):
    """Run in a child process: time the oracle on workload `name` (no GPU).

    The BLAS thread count comes from the environment the parent set before
    this interpreter (and numpy) started.  Each oracle call is timed on its
    own; the median is reported.
    """
    w = _make_workload(name, None, None, None)
    w.oracle()  # untimed: first touch of the inputs
    per = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end and len(per) < 2000:
        t0 = time.perf_counter()
        w.oracle()
        per.append(time.perf_counter() - t0)
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    print(json.dumps({"median_s": _median(per), "calls": len(per), "blas_threads": blas,
                      "nbytes": w.nbytes, "name": w.name}))


def cpu_baseline(name, budget_s=8.0):
    """The CPU oracle on the same workload, in two child processes.

    One leg with the BLAS thread count the job is given (OMP_NUM_THREADS when
    set, else every core this process may run on), one with a single thread;
    each is about budget_s of oracle calls, timed one by one (median).
    Thread counts are fixed in the child's environment before numpy loads.
    """
    import subprocess
    visible = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    threads_all = int(share) if share.isdigit() and int(share) > 0 else visible
    legs = {}
    for threads in (threads_all, 1):
        env = dict(os.environ)
        for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS",
                    "BLIS_NUM_THREADS", "NUMEXPR_NUM_THREADS"):
            env[var] = str(threads)
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-leg", name,
                            "--cpu-budget", str(budget_s)],
                           env=env, capture_output=True, text=True, timeout=budget_s * 6 + 300)
        if r.returncode != 0:
            raise RuntimeError(f"CPU oracle leg failed ({threads} threads): {r.stderr[-2000:]}")
        legs[threads] = json.loads(r.stdout.strip().splitlines()[-1])
    full, one = legs[threads_all], legs[1]
    nbytes = full["nbytes"]
    return {"value": round(nbytes / full["median_s"] / 1e9, 4), "unit": "GB/s",
            "cores": full["blas_threads"] or threads_all, "kind": "oracle",
            "sample": (f"{full['calls']} oracle calls ({full['name']}: unpack, fp64 dequantise, fp64 "
                       f"matmul), median {full['median_s'] * 1e3:.2f} ms each; the dequantise step "
                       f"runs on one thread, the matmul on the BLAS threads"),
            "single_thread": {"value": round(nbytes / one["median_s"] / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "calls": one["calls"],
                              "median_ms": round(one["median_s"] * 1e3, 3)},
            "median_ms": round(full["median_s"] * 1e3, 3),
            "host_cores_visible": visible, "cpu_model": _cpu_model()}


def _make_workload(name, wq, torch, dev):
    """The named workload (wq/torch/dev may be None when only the oracle is used)."""
    if name == "q8":
        return wl_q8(wq, torch, dev)
    if name.startswith("q8_m"):
        return wl_q8(wq, torch, dev, int(name[4:]))
    if name == "q3_f32_1024":
        return wl_q3(wq, torch, dev, 1024, 1024, "f32", 1000)
    if name.startswith("q3_f16_"):
        K, N = (int(v) for v in name[len("q3_f16_"):].split("x"))
        seed = {(4096, 4096): 1200, (4096, 11008): 1201, (11008, 4096): 1202}.get((K, N), 1203)
        return wl_q3(wq, torch, dev, K, N, "f16", seed)
    if name.startswith("q4_m"):
        return wl_q4(wq, torch, dev, int(name[4:]))
    if name.startswith("q4zp_act_m"):
        return wl_q4zp(wq, torch, dev, int(name[len("q4zp_act_m"):]), act=True)
    if name.startswith("q4zp_g64_m"):
        return wl_q4zp(wq, torch, dev, int(name[len("q4zp_g64_m"):]), 64)
    if name.startswith("q4zp_m"):
        return wl_q4zp(wq, torch, dev, int(name[len("q4zp_m"):]))
    if name.startswith("q2_m"):
        return wl_q2(wq, torch, dev, int(name[len("q2_m"):]))
    if name.startswith("q8_sep_"):        # q8_sep_f16_m512, q8_sep_f32_m512
        dt, m = name[len("q8_sep_"):].split("_m")
        return wl_q8_separated(wq, torch, dev, int(m), dt)
    if name == "w8a8":
        return wl_w8a8(wq, torch, dev)
    if name == "w8a8_smooth":
        return wl_w8a8(wq, torch, dev, smooth=True)
    if name == "w8a8_resident":
        return wl_w8a8(wq, torch, dev, resident=True)
    if name == "int8_mixed":
        return wl_int8_mixed(wq, torch, dev)
    raise SystemExit(f"unknown workload {name}")


SECONDARY = ("q3_f32_1024", "q3_f16_4096x4096", "q3_f16_4096x11008", "q3_f16_11008x4096",
             "q4_m1", "q4_m2", "q4_m4", "q4_m8", "q4_m16", "q4_m32", "q4_m64", "q4zp_m1",
             "q4zp_act_m64", "q4zp_g64_m1", "q2_m1", "q2_m8",
             "q8_m2", "q8_m8", "q8_m16", "q8_m32", "q8_m512", "q8_sep_f16_m512", "q8_sep_f32_m512",
             "w8a8", "w8a8_resident", "w8a8_smooth", "int8_mixed")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--trials", type=int, default=None,
                    help="timed trials of exactly --steps steps each (median reported); "
                         "default 11, or 5 above 500 steps")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the empty-kernel and bare-stream reference timings")
    ap.add_argument("--workload", default="q8",
                    help="q8 (headline) | q8_m* | q3_* | q4_m* | q4zp_m* | q4zp_g64_m* | q2_m* | w8a8 | w8a8_resident | w8a8_smooth | int8_mixed (single line)")
    ap.add_argument("--graph", action="store_true",
                    help="replay a captured graph of the timed steps instead of issuing them one by one")
    ap.add_argument("--stream-sweep", action="store_true",
                    help="only time the bare weight stream (wq_calib_stream_read) at 4..256 MiB and "
                         "the empty kernel, one JSON line each")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (counter calibration)")
    ap.add_argument("--cpu-leg", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-budget", type=float, default=8.0, help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_leg:
        cpu_leg(args.cpu_leg, args.cpu_budget)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 (each GPU would take its own share of the columns)"}))
        sys.exit(2)

    # The CPU oracle legs run first, in child processes, before this process
    # touches the GPU.
    cpu = (None if args.no_cpu_baseline or args.calibrate_copy or args.stream_sweep
           else cpu_baseline(args.workload))

    import torch
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        nbytes = 256 << 20
        src = torch.full((nbytes,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": nbytes,
                          "bytes_written_per_copy": nbytes, "copies": 5}))
        return
    import weight_only_quantized_dequant_amd as wq
    wq.lib()
    if args.stream_sweep:
        stream_sweep(wq, torch, dev, args.steps, args.warmup)
        return

    def make(name):
        return _make_workload(name, wq, torch, dev)

    w = make(args.workload)
    ms, R, per = time_workload(torch, w, args.steps, args.warmup, trials=args.trials,
                               method="graph" if args.graph else "eager")
    gbs = w.nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "Achieved HBM GB/s (% of 8 TB/s) for M=1 fused-dequant GEMV, K=N=4096",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": getattr(w, "dtype", "see workload"), "data": "synthetic (seeded: N(0,1) activations, N(0,0.02) weights quantised offline)",
        "config": dict(getattr(w, "config", {"workload": w.name}), rotation_copies=R,
                       pct_of_hbm_peak=round(100 * gbs / HBM_PEAK_GBS, 2)),
        "timing": {"trials": len(per), "steps_per_trial": args.steps, "statistic": "median",
                   "per_trial_us_per_step": [round(t * 1e3, 3) for t in per],
                   "method": ("HIP events around exactly `steps` calls on the launch stream, queued "
                              "behind a spin kernel, after a pre-roll of one call per rotated copy"
                              if not args.graph else
                              "HIP events around one replay of a graph of exactly `steps` calls, "
                              "after a pre-roll of one call per rotated copy")},
    }
    kern = "q8_group" if args.workload == "q8" else None
    traffic = committed_traffic(kern, "4096") if kern else None
    out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                       "algorithmic_bytes_per_launch": w.nbytes}
    if args.workload == "q8" and not args.no_calibration:
        out["calibration"] = calibration(wq, torch, w, args.steps, args.warmup, ms)
    if not args.headline_only:
        sec = {}
        for name in SECONDARY:
            sw = make(name)
            big = name.startswith("w8a8") or name == "int8_mixed"
            st, wu = (100, 10) if big else (300, 30)
            sms, sR, _ = time_workload(torch, sw, st, wu, trials=5)
            e = {"us_per_call": round(sms * 1e3, 3), "GB_per_s": round(sw.nbytes / (sms * 1e-3) / 1e9, 1),
                 "pct_hbm_peak": round(100 * sw.nbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                 "rotation_copies": sR, "algorithmic_bytes": sw.nbytes}
            if not args.no_calibration:
                # The same rotation, a kernel that only reads each copy's weight
                # (slot 1 of every argument set) once: the time any kernel that
                # moves those bytes needs here.
                sink = torch.zeros(1, dtype=torch.int32, device=dev)
                ref = Workload("weight stream", sw.nbytes, sw.make,
                               lambda c: wq.calib_stream_read(c[1], sink))
                rms, _, _ = time_workload(torch, ref, st, wu, trials=5)
                e["weight_stream_us"] = round(rms * 1e3, 3)
                e["share_of_stream_ceiling"] = round(rms / sms, 4)
            if sw.flops:
                e["TOPS"] = round(sw.flops / (sms * 1e-3) / 1e12, 1)
                e["pct_mfma_peak"] = round(100 * sw.flops / (sms * 1e-3) / 1e12 / sw.peak_tops, 2)
            sec[sw.name] = e
            del sw
        out["secondary"] = sec
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out))


if __name__ == "__main__":
    main()
