"""Throughput of the fused W4A16 layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all]

A step is one call of the fused layer (awq_gemv at M = 1) on the decode
workload: the Llama-3-8B MLP gate shape, M=1, K=4096, N=14336, group 128,
asymmetric zero points.  The layer is packed once (as when a checkpoint is
loaded); each step streams the packed weight, unpacks, dequantizes, multiplies,
reduces and writes Y.  The weight is replicated into enough copies (>= 1 GiB)
that successive steps read different copies, so every step streams from HBM
rather than from the 256 MB last-level cache.  Inputs are resident in HBM before
the timed region.  The K timed steps are launched as one captured HIP graph on
one stream and bracketed by events on that stream.

Prints one JSON line: value = algorithmic bytes per step / time per step, in
GB/s.  Also reported: the roofline of the dominant kernel (awq_gemv), the
batched GEMM (awq_gemm, prefill shape M=2048) in TFLOP/s, and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 flop/clk/CU, dense fp16
METRIC = "W4A16 GEMV HBM GB/s (% of peak) at M=1; GEMM TFLOP/s (% MFMA peak) at M=2048"
ROTATE_BYTES = 1 << 30


def alg_bytes(w, M):
    """Bytes that must cross HBM once: packed weight, scales, zeros, X, Y."""
    zeros = 0 if w.symmetric else w.N * w.K // (2 * w.G)
    return w.K * w.N // 2 + 2 * w.N * (w.K // w.G) + zeros + 2 * M * w.K + 2 * M * w.N


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.float16) if a.dtype == np.uint16 \
        else torch.from_numpy(a)
    return t.to("cuda")


def build_layers(w, copies):
    """The workload's layer packed on the GPU, then replicated ``copies`` times."""
    from w4a16_group_quantized_amd import binding, synth
    import torch
    _, codes, zeros, scales = synth.workload_inputs(w, M=1)
    base = binding.make_layer(to_dev(codes), None if zeros is None else to_dev(zeros),
                              to_dev(scales), w.G)
    layers = [base]
    for _ in range(copies - 1):
        layers.append(binding.Layer(base.qweight.clone(), base.scales.clone(),
                                    None if base.qzeros is None else base.qzeros.clone(),
                                    base.K, base.N, base.group_size))
    torch.cuda.synchronize()
    return layers


def time_calls(fn_name, x, layers, y, steps, warmup):
    """Launches ``steps`` calls, cycling through ``layers``, as one HIP graph on
    one stream; returns seconds per call measured with events on that stream."""
    import torch
    from w4a16_group_quantized_amd import binding

    stream = torch.cuda.Stream()
    fn = getattr(binding, fn_name)
    with torch.cuda.stream(stream):
        for i in range(max(warmup, 1)):
            fn(x, layers[i % len(layers)], out=y)
    stream.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            fn(x, layers[i % len(layers)], out=y)
    with torch.cuda.stream(stream):
        graph.replay()          # first replay uploads the graph: untimed
    stream.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        graph.replay()
        end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3 / steps


def bench_gemv(name, steps, warmup):
    import torch
    from w4a16_group_quantized_amd import synth
    w = synth.WORKLOADS[name]
    per_copy = alg_bytes(w, 0)
    copies = max(2, math.ceil(ROTATE_BYTES / per_copy))
    layers = build_layers(w, copies)
    X = to_dev(synth.make_x(w.M, w.K, w.wid, w.n_outliers, w.outlier_gain))
    y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    t = time_calls("gemv", X, layers, y, steps, warmup)
    b = alg_bytes(w, w.M)
    del layers
    torch.cuda.empty_cache()
    return {"workload": name, "M": w.M, "K": w.K, "N": w.N, "group_size": w.G,
            "symmetric": w.symmetric, "entry": "awq_gemv", "weight_copies": copies,
            "us_per_call": t * 1e6, "alg_bytes": b, "gbs": b / t / 1e9,
            "hbm_frac": b / t / 1e9 / HBM_PEAK_GBS}


def bench_gemm(name, steps, warmup):
    import torch
    from w4a16_group_quantized_amd import synth
    w = synth.WORKLOADS[name]
    layers = build_layers(w, 1)
    X = to_dev(synth.make_x(w.M, w.K, w.wid, w.n_outliers, w.outlier_gain))
    y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    t = time_calls("gemm", X, layers, y, steps, warmup)
    flops = 2.0 * w.M * w.N * w.K
    del layers
    torch.cuda.empty_cache()
    return {"workload": name, "M": w.M, "K": w.K, "N": w.N, "group_size": w.G,
            "symmetric": w.symmetric, "entry": "awq_gemm", "us_per_call": t * 1e6,
            "tflops": flops / t / 1e12, "mfma_frac": flops / t / 1e12 / MFMA_F16_PEAK_TFLOPS}


def cpu_baseline(name, budget_s=10.0):
    """The oracle as it stands, single threaded, from packed inputs to Y, repeated
    over the whole decode layer until ``budget_s`` seconds have passed."""
    import oracle
    from w4a16_group_quantized_amd import synth
    w = synth.WORKLOADS[name]
    X, codes, zeros, scales = synth.workload_inputs(w)
    o = oracle.load()
    Q, QZ = o.pack(codes), (None if zeros is None else o.pack_zeros(zeros))
    runs, t0 = 0, time.perf_counter()
    while True:
        o.linear(X, Q, scales, QZ, w.G)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / runs
    return {"value": alg_bytes(w, w.M) / per / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{runs} full passes of the {name} layer (M={w.M} K={w.K} N={w.N}), "
                      f"unpack + exact dequant + fp64 matmul, {per:.2f} s each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--all", action="store_true", help="also time the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards by output columns with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    from w4a16_group_quantized_amd import binding
    binding.load()

    head = bench_gemv("decode_8b_gate", args.steps, args.warmup)
    gemm = bench_gemm("prefill_out_proj", max(10, args.steps // 10), max(2, args.warmup // 10))
    extra = []
    if args.all:
        extra.append(bench_gemv("gate_up_m16", args.steps, args.warmup))
        extra.append(bench_gemv("sym70b_m1", args.steps, args.warmup))
        extra.append(bench_gemm("gate_up_m16", args.steps, args.warmup))
        extra.append(bench_gemm("sym70b_m4096", max(5, args.steps // 40), 2))

    out = {
        "metric": METRIC,
        "value": round(head["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_call"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "decode_8b_gate", "M": 1, "K": 4096, "N": 14336, "group_size": 128,
                   "symmetric": False, "entry": "awq_gemv", "weight_copies": head["weight_copies"],
                   "launch": "hip_graph"},
        "roofline": {"bound": "hbm", "achieved": round(head["gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(head["hbm_frac"], 4), "traffic": None},
        "gemm": {"workload": gemm["workload"], "M": gemm["M"], "K": gemm["K"], "N": gemm["N"],
                 "tflops": round(gemm["tflops"], 1), "peak": MFMA_F16_PEAK_TFLOPS,
                 "frac": round(gemm["mfma_frac"], 4), "us_per_call": round(gemm["us_per_call"], 2)},
    }
    if extra:
        out["extra"] = extra
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline("decode_8b_gate")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
