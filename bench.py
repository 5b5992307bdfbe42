"""Throughput of the fused W4A16 layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all]

A step is one call of the fused layer (awq_gemv at M = 1) on the decode
workload: the Llama-3-8B MLP gate shape, M=1, K=4096, N=14336, group 128,
asymmetric zero points.  The layer is packed once and its words repacked
into the library's blocked layout (as when a checkpoint is loaded; --layout
canonical keeps awq_pack's word order, --layout interleaved the interleaved
nibbles without the blocks); each step streams the packed
weight, unpacks, dequantizes, multiplies,
reduces and writes Y.  The weight is replicated into enough copies (>= 1 GiB)
that successive steps read different copies, so every step streams from HBM
rather than from the 256 MB last-level cache.  Inputs are resident in HBM before
the timed region.  The K timed steps are launched as one captured HIP graph on
one stream and bracketed by events on that stream, with the device synchronized
before and after; that replay gives the value.  Four more replays of the same
graph give the median, minimum and maximum time per call ("timing").  With
--all, the same calls on a single cache-resident copy ("hot_cache_us") are
timed too, as context; the default run times only cold calls, so that a
kernel-trace profile of it averages the same calls the value comes from.

Prints one JSON line: value = algorithmic bytes per step / time per step, in
GB/s.  Also reported:
* roofline: the dominant kernel (awq_gemv's decode kernel) against 8 TB/s;
* gemm: the batched GEMM (awq_gemm, prefill shape M=2048) in TFLOP/s against
  the fp16 MFMA peak;
* configs: every workload configuration, each timed the same way on its entry
  points -- the tiny layer (launch-bound), the decode layer, the fused gate/up
  layer at 16 rows through awq_gemv, awq_gemv_gate_up and awq_gemm (the
  GEMV/GEMM crossover), the prefill GEMM, and the 70B-shape layer at 1 row
  (awq_gemv) and 4096 rows (awq_gemm) -- with the fraction of the roofline
  that bounds each;
* context: torch.matmul (hipBLASLt) on a plain fp16 weight of the prefill
  shape, not the metric;
* cpu_baseline: the oracle at every configuration on one host thread and on
  all of them (bit-identical outputs), the 70B-shape batch from its first 64
  rows scaled by M / 64; value is the decode layer on all host threads.

Profiling helpers (the figures under profiles/ come from these):

    python bench.py --profile gemv|gemv16|gemm
        a short fixed sequence for rocprofv3 counter passes: 20 calls of the
        kernel on its workload (gemv: awq_gemv on the decode layer; gemv16:
        awq_gemv on the fused gate/up layer's 16 rows; gemm: awq_gemm on the
        prefill layer), each its own dispatch, then 5 device copies of 64 MiB
        -- the plain copy kernel that calibrates FETCH_SIZE/WRITE_SIZE
    python bench.py --summarize-pmc OUT DIR...
        folds the counter CSVs of rocprofv3 --pmc runs into a text summary with
        per-dispatch medians, the copy calibration, the HBM traffic per launch
        and the hash of the kernel's sources
    python bench.py --summarize-stats OUT DIR
        the same for a rocprofv3 --kernel-trace --stats run

The roofline's "traffic" is read from the committed counter summary of the
GEMV kernel, and only while the hash of its sources still matches.

    python bench.py --ceilings
        only the two ceilings below, as one JSON line

"ceilings" in the JSON line (context, not the metric) are what this part
sustains on the two bound resources, measured live by the probes in
probes/ (beside this file): a plain streaming read of the decode layer's
byte count from the same number of cold copies (the floor for any kernel that
must read those bytes once), and fp16 MFMA chains on operands that change every
instruction (the matrix cores' rate once the clock has dropped to the power
budget, which data-free peaks hide).  Each kernel's fraction of its ceiling is
reported beside the fraction of the vendor peak.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 flop/clk/CU, dense fp16
METRIC = "W4A16 GEMV HBM GB/s (% of peak) at M=1; GEMM TFLOP/s (% MFMA peak) at M=2048"
ROTATE_BYTES = 1 << 30
# Graph replays per configuration line; the line reports their median, so that
# one slow replay does not decide it.
CONFIG_REPS = 5
GEMM_SETTLE_S = 0.1            # untimed replays before an MFMA-bound timing (see time_calls)
CALIBRATION_COPY_BYTES = 64 << 20
PROFILE_CALLS = 20
CSRC = os.path.join(ROOT, "w4a16_group_quantized_amd", "csrc")
# Sources that define each profiled kernel (the launcher declarations in
# awq_internal.h generate no code), and the build script that sets its compile
# flags: a counter summary is valid only for them.
KERNEL_SOURCES = {
    "gemv": ["awq_gemv_kernels.h", "awq_device.h", "../build.py"],
    "gemm": ["awq_gemm_kernels.h", "awq_device.h", "../build.py"],
}
KERNEL_SOURCES["gemv16"] = KERNEL_SOURCES["gemv"]
KERNEL_NAMES = {"gemv": ("stream_kernel", "fold_kernel", "exact_kernel"), "gemm": ("gemm_kernel", "mfma32_kernel")}
KERNEL_NAMES["gemv16"] = KERNEL_NAMES["gemv"]
# --profile kinds: the workload and the binding entry of each (gemv16: the fused
# gate/up layer's 16 rows through awq_gemv)
PROFILE_WORKLOAD = {"gemv": "decode_8b_gate", "gemm": "prefill_out_proj", "gemv16": "gate_up_m16"}
PROFILE_ENTRY = {"gemv": "gemv", "gemm": "gemm", "gemv16": "gemv"}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "awq_gemv_decode_8b_gate_counters.txt")
GEMM_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "awq_gemm_prefill_out_proj_counters.txt")


def source_hash(kind):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


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


# qweight layout of every benchmarked layer (--layout): canonical, or one of the
# kernel-private ones, interleaved or blocked (repacked once after packing, as
# at load time).
LAYOUT = {"canonical": 0, "interleaved": 1, "blocked": 2}
BENCH_LAYOUT = "blocked"


def build_layers(w, copies):
    """The workload's layer packed on the GPU (repacked to BENCH_LAYOUT), then
    replicated ``copies`` times."""
    from w4a16_group_quantized_amd import binding, synth
    import torch
    _, codes, zeros, scales = synth.workload_inputs(w, M=1)
    base = binding.make_layer(to_dev(codes), None if zeros is None else to_dev(zeros),
                              to_dev(scales), w.G)
    if LAYOUT[BENCH_LAYOUT] != base.layout:
        base = binding.repack(base, LAYOUT[BENCH_LAYOUT])
    layers = [base]
    for _ in range(copies - 1):
        layers.append(binding.Layer(base.qweight.clone(), base.scales.clone(),
                                    None if base.qzeros is None else base.qzeros.clone(),
                                    base.K, base.N, base.group_size, base.layout))
    torch.cuda.synchronize()
    return layers


def time_calls(fn_name, x, layers, y, steps, warmup, reps=1, settle_s=0.0):
    """Launches ``steps`` calls, cycling through ``layers``, as one HIP graph on
    one stream; returns seconds per call of the first timed replay, measured
    with events on that stream between device synchronizations.  With reps > 1
    the graph is replayed reps times in all and (first, median, min, max) is
    returned.  ``settle_s`` > 0 replays the graph, untimed, for that long first:
    under sustained MFMA load the GPU's clock settles only after some 25 ms (the
    prefill GEMM runs 69, 65, then 60.6 us per call in its first three 13 ms
    rounds), so the GEMMs are timed at that steady state."""
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
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        with torch.cuda.stream(stream):
            start.record(stream)
            graph.replay()
            end.record(stream)
        end.synchronize()
        times.append(start.elapsed_time(end) * 1e-3 / steps)
    torch.cuda.synchronize()
    if reps == 1:
        return times[0]
    return times[0], statistics.median(times), min(times), max(times)


def bench_gemv(name, steps, warmup, reps=1, hot=False, max_copies=None):
    """awq_gemv on the workload, cycling through enough weight copies that every
    call reads HBM; ``reps`` replays give the median (and min, max); ``hot``
    adds the same calls on one copy (cache-resident), as context.
    ``max_copies`` caps the copies (the tiny layer: launch-bound, cache-resident)."""
    import torch
    from w4a16_group_quantized_amd import synth
    w = synth.WORKLOADS[name]
    per_copy = alg_bytes(w, 0)
    copies = max(2, math.ceil(ROTATE_BYTES / per_copy))
    if max_copies is not None:
        copies = min(copies, max_copies)
    layers = build_layers(w, copies)
    X = to_dev(synth.make_x(w.M, w.K, w.wid, w.n_outliers, w.outlier_gain))
    y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    r = time_calls("gemv", X, layers, y, steps, warmup, reps)
    t, t_med, t_min, t_max = r if reps > 1 else (r, r, r, r)
    t_hot = time_calls("gemv", X, layers[:1], y, steps, warmup) if hot else None
    b = alg_bytes(w, w.M)
    del layers
    torch.cuda.empty_cache()
    out = {"workload": name, "M": w.M, "K": w.K, "N": w.N, "group_size": w.G,
           "symmetric": w.symmetric, "entry": "awq_gemv", "weight_copies": copies,
           "us_per_call": t * 1e6, "alg_bytes": b, "gbs": b / t / 1e9,
           "hbm_frac": b / t / 1e9 / HBM_PEAK_GBS}
    if reps > 1:
        out["reps"] = {"n": reps, "calls_each": steps, "median_us": t_med * 1e6,
                       "min_us": t_min * 1e6, "max_us": t_max * 1e6}
    if hot:
        out["hot_cache_us"] = t_hot * 1e6
    return out


def bench_gate_up(name, M, steps, warmup, reps=CONFIG_REPS):
    """awq_gemv_gate_up on a concatenated [gate | up] layer: h = SiLU(gate) * up;
    the median of ``reps`` replays."""
    import torch
    from w4a16_group_quantized_amd import synth
    w = synth.WORKLOADS[name]
    copies = max(2, math.ceil(ROTATE_BYTES / alg_bytes(w, 0)))
    layers = build_layers(w, copies)
    X = synth.make_x(max(M, w.M), w.K, w.wid, w.n_outliers, w.outlier_gain)[:M]
    X = to_dev(np.ascontiguousarray(X))
    h = torch.empty((M, w.N // 2), dtype=torch.float16, device="cuda")
    t = time_calls("gemv_gate_up", X, layers, h, steps, warmup, reps)
    t = t[1] if reps > 1 else t                                # the median
    b = alg_bytes(w, M) - 2 * M * w.N + 2 * M * (w.N // 2)   # h replaces Y
    del layers
    torch.cuda.empty_cache()
    return {"workload": name, "M": M, "K": w.K, "N": w.N, "group_size": w.G,
            "symmetric": w.symmetric, "entry": "awq_gemv_gate_up", "weight_copies": copies,
            "replays": reps, "us_per_call": t * 1e6, "alg_bytes": b, "gbs": b / t / 1e9,
            "hbm_frac": b / t / 1e9 / HBM_PEAK_GBS}


def bench_gemm_gate_up(name, M, steps, warmup):
    """awq_gemm_gate_up at batch M on a concatenated [gate | up] layer."""
    import torch
    from w4a16_group_quantized_amd import synth
    w = synth.WORKLOADS[name]
    layers = build_layers(w, 1)
    X = to_dev(synth.make_x(M, w.K, w.wid, w.n_outliers, w.outlier_gain))
    h = torch.empty((M, w.N // 2), dtype=torch.float16, device="cuda")
    t = time_calls("gemm_gate_up", X, layers, h, steps, warmup, settle_s=GEMM_SETTLE_S)
    flops = 2.0 * M * w.N * w.K
    del layers
    torch.cuda.empty_cache()
    return {"workload": name, "M": M, "K": w.K, "N": w.N, "group_size": w.G,
            "symmetric": w.symmetric, "entry": "awq_gemm_gate_up", "us_per_call": t * 1e6,
            "tflops": flops / t / 1e12, "mfma_frac": flops / t / 1e12 / MFMA_F16_PEAK_TFLOPS}


def bench_quantize(name, steps, warmup):
    """awq_quantize on a layer of the workload's shape: fp16 W -> packed codes,
    scales, zero points, cycling through enough copies of W (1 GiB) that every
    call reads HBM.  Algorithmic bytes: W read once, the layer written."""
    import torch
    from w4a16_group_quantized_amd import binding, synth
    w = synth.WORKLOADS[name]
    rng = np.random.default_rng(w.wid)
    W0 = torch.from_numpy((rng.standard_normal((w.K, w.N)) * 0.02).astype(np.float16)).cuda()
    copies = max(2, math.ceil(ROTATE_BYTES / (2 * w.K * w.N)))
    Ws = [W0.clone() for _ in range(copies)]
    for i in range(max(warmup, 1)):
        binding.quantize(Ws[i % copies], w.G, w.symmetric)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        binding.quantize(Ws[i % copies], w.G, w.symmetric)
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / steps
    b = 2 * w.K * w.N + alg_bytes(w, 0)
    del Ws, W0
    torch.cuda.empty_cache()
    return {"workload": name, "entry": "awq_quantize", "K": w.K, "N": w.N, "group_size": w.G,
            "w_copies": copies, "us_per_call": t * 1e6, "alg_bytes": b, "gbs": b / t / 1e9,
            "hbm_frac": b / t / 1e9 / HBM_PEAK_GBS}


def bench_gemm_splitk(name, M, steps, warmup):
    """awq_gemm and awq_gemm_splitk (slices chosen automatically) at batch M on the
    workload's layer, as one captured graph each."""
    import dataclasses
    import torch
    from w4a16_group_quantized_amd import binding, synth
    w = dataclasses.replace(synth.WORKLOADS[name], M=M)
    layers = build_layers(w, 1)
    x = to_dev(synth.make_x(M, w.K, w.wid, w.n_outliers, w.outlier_gain))
    y = torch.empty((M, w.N), dtype=torch.float16, device="cuda")
    t_plain = time_calls("gemm", x, layers, y, steps, warmup)
    splits = binding.splitk_splits(M, layers[0])
    ws = torch.empty(max(binding.load().awq_gemm_splitk_workspace_bytes(M, w.N, splits), 16),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(max(warmup, 1)):
            binding.gemm_splitk(x, layers[0], splits, out=y, stream=stream, workspace=ws)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(steps):
            binding.gemm_splitk(x, layers[0], splits, out=y, stream=stream, workspace=ws)
    with torch.cuda.stream(stream):
        graph.replay()
    stream.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / steps
    flops = 2.0 * M * w.N * w.K
    return {"workload": name, "entry": "awq_gemm_splitk", "M": M, "K": w.K, "N": w.N,
            "splits": splits, "us_per_call": t * 1e6, "tflops": flops / t / 1e12,
            "awq_gemm_us": t_plain * 1e6}


def bench_scale_search(name, M, n_alpha, reps):
    """awq_scale_search on the workload's layer shape: M calibration rows (X ~ N(0, 1)
    with the workload's outlier channels), an fp16 W ~ N(0, 0.02), an evenly spaced
    grid of n_alpha values in [0, 1).  Each candidate quantizes the migrated weight,
    runs the fused GEMM and reduces the error; the fp16 reference GEMM runs once."""
    import torch
    from w4a16_group_quantized_amd import binding, synth
    w = synth.WORKLOADS[name]
    x = to_dev(synth.make_x(M, w.K, w.wid, max(w.n_outliers, w.K // 100), 20.0))
    rng = np.random.default_rng(w.wid)
    W = torch.from_numpy((rng.standard_normal((w.K, w.N)) * 0.02).astype(np.float16)).cuda()
    alphas = [i / n_alpha for i in range(n_alpha)]
    lib = binding.load()
    ws = torch.empty(lib.awq_scale_search_workspace_bytes(M, w.K, w.N, w.G), dtype=torch.uint8,
                     device="cuda")
    binding.scale_search(x, W, w.G, alphas, w.symmetric, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        best, _, _ = binding.scale_search(x, W, w.G, alphas, w.symmetric, workspace=ws)
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    flops = 2.0 * M * w.N * w.K * (n_alpha + 1)    # the candidates' GEMMs and the reference
    return {"workload": name, "entry": "awq_scale_search", "M": M, "K": w.K, "N": w.N,
            "group_size": w.G, "n_alpha": n_alpha, "ms_per_search": t * 1e3,
            "us_per_candidate": t * 1e6 / n_alpha, "gemm_tflops": flops / t / 1e12,
            "best_alpha": alphas[int(best.item())]}


def torch_matmul_context(name, steps):
    """Not the metric: torch.matmul (the vendor fp16 GEMM) on the dequantized
    weight of the same shape, for context on what a plain fp16 GEMM reaches."""
    import torch
    from w4a16_group_quantized_amd import synth
    w = synth.WORKLOADS[name]
    a = torch.randn(w.M, w.K, dtype=torch.float16, device="cuda")
    b = torch.randn(w.K, w.N, dtype=torch.float16, device="cuda") * 0.01
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        a @ b
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / steps
    flops = 2.0 * w.M * w.N * w.K
    return {"workload": name, "entry": "torch.matmul fp16 (context, not the metric)",
            "us_per_call": t * 1e6, "tflops": flops / t / 1e12}


def _probes():
    import ctypes
    import probes
    if not os.path.exists(probes.LIBRARY):
        raise RuntimeError(f"{probes.LIBRARY} is not built (run `python -m probes` first)")
    lib = ctypes.CDLL(probes.LIBRARY)
    lib.awq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.awq_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    return lib


def ceiling_read(name, steps=200):
    """A plain streaming read of the workload's weight bytes, cycling through
    as many copies as the GEMV bench uses, launched as one HIP graph; the best
    of three grid sizes."""
    import torch
    from w4a16_group_quantized_amd import synth
    lib = _probes()
    w = synth.WORKLOADS[name]
    nbytes = alg_bytes(w, 0) // 16 * 16
    copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
    bufs = [torch.full((nbytes,), i, dtype=torch.uint8, device="cuda") for i in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    best = None
    for blocks in (1024, 2048, 4096):
        stream = torch.cuda.Stream()

        def call(i):
            rc = lib.awq_probe_stream_read(bufs[i % copies].data_ptr(), nbytes, blocks,
                                           sink.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"awq_probe_stream_read failed: hip error {rc}")
        with torch.cuda.stream(stream):
            for i in range(20):
                call(i)
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                call(i)
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        e1.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / steps
        if best is None or t < best[0]:
            best = (t, blocks)
        del graph
    del bufs
    torch.cuda.empty_cache()
    t, blocks = best
    return {"kernel": "streaming read, 16-byte non-temporal loads, grid-stride",
            "bytes": nbytes, "copies": copies, "blocks": blocks, "us_per_call": round(t * 1e6, 3),
            "gbs": round(nbytes / t / 1e9, 1)}


def ceiling_mfma(blocks=1024, iters=4000, reps=5):
    """v_mfma_f32_32x32x16_f16 chains on seeded random operands, all CUs busy."""
    import torch
    lib = _probes()
    rng = np.random.default_rng(2024)
    ops = to_dev(rng.uniform(-1.0, 1.0, 512).astype(np.float16).view(np.uint16))
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def call():
        rc = lib.awq_probe_mfma(ops.data_ptr(), out.data_ptr(), blocks, iters, stream)
        if rc != 0:
            raise RuntimeError(f"awq_probe_mfma failed: hip error {rc}")
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    flops = blocks * 4.0 * iters * 8 * 32768.0
    return {"kernel": "32x32x16 fp16 MFMA chains, random operands changing every instruction",
            "blocks": blocks, "tflops": round(flops / t / 1e12, 1),
            "frac_of_peak": round(flops / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}


def bench_gemm(name, steps, warmup, rotate=False, reps=CONFIG_REPS):
    """awq_gemm on the workload, the median of ``reps`` replays; ``rotate``
    cycles through weight copies (1 GiB) as the GEMV bench does, for batches
    small enough to be HBM-bound."""
    import torch
    from w4a16_group_quantized_amd import synth
    w = synth.WORKLOADS[name]
    copies = max(2, math.ceil(ROTATE_BYTES / alg_bytes(w, 0))) if rotate else 1
    layers = build_layers(w, copies)
    X = to_dev(synth.make_x(w.M, w.K, w.wid, w.n_outliers, w.outlier_gain))
    y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    t = time_calls("gemm", X, layers, y, steps, warmup, reps, settle_s=GEMM_SETTLE_S)
    t = t[1] if reps > 1 else t                                # the median
    flops = 2.0 * w.M * w.N * w.K
    del layers
    torch.cuda.empty_cache()
    return {"workload": name, "M": w.M, "K": w.K, "N": w.N, "group_size": w.G,
            "symmetric": w.symmetric, "entry": "awq_gemm", "us_per_call": t * 1e6,
            "weight_copies": copies, "replays": reps,
            "tflops": flops / t / 1e12, "mfma_frac": flops / t / 1e12 / MFMA_F16_PEAK_TFLOPS}


# The oracle's timed samples, one per configuration: (configuration, workload,
# rows timed or None for all of them).  The 70B-shape batch is timed on its
# first 64 rows and scaled by M / 64: rows are independent.
CPU_SAMPLES = (("cfg1", "tiny", None), ("cfg2", "decode_8b_gate", None),
               ("cfg3", "gate_up_m16", None), ("cfg4", "prefill_out_proj", None),
               ("cfg5a", "sym70b_m1", None), ("cfg5b", "sym70b_m4096", 64))


def host_threads():
    """Host threads this process may run on (the machine's CPU share)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(min_s=1.0):
    """The oracle as it stands, from packed inputs to Y (unpack, exact dequant,
    fp64 matmul), on one thread and on all host threads, at every configuration.

    All threads run the same oracle over column slices of the layer: each
    column keeps its increasing-k sum, so the outputs are bit-identical to the
    single-threaded run (checked here).  Each setting repeats whole passes for
    at least ``min_s`` seconds (one pass for the large configurations).  The
    headline value is the decode layer on all host threads."""
    import oracle
    from w4a16_group_quantized_amd import synth
    o = oracle.load()
    threads = host_threads()
    results = []
    for cfg, name, rows in CPU_SAMPLES:
        w = synth.WORKLOADS[name]
        X, codes, zeros, scales = synth.workload_inputs(w, M=rows)
        Q, QZ = o.pack(codes), (None if zeros is None else o.pack_zeros(zeros))
        scale = w.M / X.shape[0]
        entry = {"config": cfg, "workload": name, "M": w.M, "K": w.K, "N": w.N,
                 "rows_timed": X.shape[0]}
        if scale != 1:
            entry["extrapolated"] = f"{X.shape[0]} of {w.M} rows timed, x{scale:g}; rows independent"
        outs = []
        for th in (1, threads):
            passes, t0 = 0, time.perf_counter()
            while True:
                y64, y16 = o.linear_columns(X, Q, scales, QZ, w.G, th)
                passes += 1
                el = time.perf_counter() - t0
                if el >= min_s:
                    break
            outs.append(y16)
            per = el / passes * scale
            key = "one_thread" if th == 1 else "all_threads"
            rec = {"threads": th, "passes": passes, "s_per_call": round(per, 4)}
            if w.M <= 16:
                rec["gbs"] = round(alg_bytes(w, w.M) / per / 1e9, 4)
            else:
                rec["tflops"] = round(2.0 * w.M * w.N * w.K / per / 1e12, 6)
            entry[key] = rec
        entry["bits_identical"] = bool(np.array_equal(outs[0], outs[1]))
        results.append(entry)
    head = next(e for e in results if e["workload"] == "decode_8b_gate")
    return {"value": head["all_threads"]["gbs"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"full passes of the decode_8b_gate layer (M=1 K=4096 N=14336) on {threads} "
                      f"host threads over column slices, unpack + exact dequant + fp64 matmul, "
                      f"{head['all_threads']['s_per_call']:.3f} s each "
                      f"({head['one_thread']['s_per_call']:.3f} s on one thread); "
                      f"every configuration below at 1 and {threads} threads",
            "single_thread": {"value": head["one_thread"]["gbs"], "unit": "GB/s", "cores": 1},
            "configs": results,
            "host": {"cpu": host_cpu_model(), "nproc": os.cpu_count(), "threads": threads}}


def host_cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def profile_run(kind):
    """Fixed dispatch sequence for counter passes (see the module docstring)."""
    import torch
    from w4a16_group_quantized_amd import binding, synth
    binding.load()
    name = PROFILE_WORKLOAD[kind]
    w = synth.WORKLOADS[name]
    copies = max(2, math.ceil(ROTATE_BYTES / alg_bytes(w, 0))) if kind != "gemm" else 1
    layers = build_layers(w, copies)
    X = to_dev(synth.make_x(w.M, w.K, w.wid, w.n_outliers, w.outlier_gain))
    y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    fn = getattr(binding, PROFILE_ENTRY[kind])
    for i in range(PROFILE_CALLS):
        fn(X, layers[i % copies], out=y)
    torch.cuda.synchronize()
    a = torch.ones(CALIBRATION_COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"profiled {PROFILE_CALLS} x awq_{PROFILE_ENTRY[kind]} on {name}, then 5 copies of "
          f"{CALIBRATION_COPY_BYTES} bytes", flush=True)


def _per_dispatch(dirs):
    """{kernel: {counter: [value per dispatch]}} from rocprofv3 --pmc CSVs."""
    out = {}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            acc, dur = {}, {}
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    k = row["Kernel_Name"]
                    if row.get("Start_Timestamp") and row.get("End_Timestamp"):
                        dur[(k, row["Dispatch_Id"])] = (float(row["End_Timestamp"]) -
                                                        float(row["Start_Timestamp"]))
                    c = row["Counter_Name"]
                    key = (k, c, row["Dispatch_Id"])
                    v = float(row["Counter_Value"])
                    # GRBM counters are per XCD and count the same clock on
                    # each: take the largest; every other counter is summed
                    # over its instances
                    acc[key] = max(acc.get(key, 0.0), v) if c.startswith("GRBM_") else acc.get(key, 0.0) + v
            for (k, c, did), v in acc.items():
                out.setdefault(k, {}).setdefault(c, []).append((int(did), v))
            for (k, did), ns in dur.items():
                out.setdefault(k, {}).setdefault("duration_ns", []).append((int(did), ns))
    for per in out.values():
        for c in per:
            per[c].sort()
    return out


def _short(kernel):
    k = kernel.replace("void ", "").replace("(anonymous namespace)", "anon")
    return k.split("(")[0][:90]


def summarize_pmc(out_path, dirs, kind, commands):
    data = _per_dispatch(dirs)
    kern = [k for k in data if any(n in k for n in KERNEL_NAMES[kind])]
    copyk = [k for k in data if "copyBuffer" in k]
    lines = [f"# rocprofv3 --pmc counters: awq_{PROFILE_ENTRY[kind]} on {PROFILE_WORKLOAD[kind]}",
             "# commands (each a run of its own):"]
    lines += [f"#   {c}" for c in commands]
    lines.append(f"# source_sha256: {source_hash(kind)}")
    lines.append("# per kernel and counter: median over dispatches of the per-dispatch sum")
    lines.append(f"{'kernel':90s} {'counter':28s} {'median':>14s} {'dispatches':>10s}")
    med = {}
    for k in kern + copyk:
        for c, vals in sorted(data[k].items()):
            if k in copyk:
                vals = vals[-5:]     # the calibration copies end the profiled sequence
            m = statistics.median(v for _, v in vals)
            med[(k, c)] = m
            lines.append(f"{_short(k):90s} {c:28s} {m:14.1f} {len(vals):10d}")
    traffic = None
    if kern and copyk:
        ck = copyk[0]
        facs = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if (ck, c) in med and med[(ck, c)] > 0:
                facs[c] = CALIBRATION_COPY_BYTES / (med[(ck, c)] * 1024.0)
        if len(facs) == 2 and all((kern[0], c) in med for c in facs):
            for c, f in facs.items():
                lines.append(f"calibration {c}: copy of {CALIBRATION_COPY_BYTES} bytes reads "
                             f"{med[(ck, c)]:.1f} KiB -> factor {f:.4f}")
            traffic = sum(med[(kern[0], c)] * 1024.0 * f for c, f in facs.items())
            lines.append(f"traffic_bytes_per_launch: {traffic:.0f}")
    if kern and all((kern[0], c) in med for c in ("SQ_BUSY_CYCLES", "duration_ns")):
        # SQ_BUSY_CYCLES counts, per shader engine (32: 8 XCDs x 4), the clock
        # cycles in which it holds a wave of the dispatch: the kernel's length
        # in shader clocks
        se_cycles = med[(kern[0], "SQ_BUSY_CYCLES")] / 32.0
        lines.append(f"shader_clock_ghz: {se_cycles / med[(kern[0], 'duration_ns')]:.3f} "
                     f"(SQ_BUSY_CYCLES / 32 shader engines / dispatch duration)")
        if (kern[0], "SQ_VALU_MFMA_BUSY_CYCLES") in med:
            # matrix-core busy cycles per SIMD (1024: 256 CUs x 4) over those cycles
            simd_busy = med[(kern[0], "SQ_VALU_MFMA_BUSY_CYCLES")] / 1024.0
            lines.append(f"mfma_busy_frac: {simd_busy / se_cycles:.4f} "
                         f"(SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (SQ_BUSY_CYCLES / 32))")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_stats(out_path, d, command):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    lines = ["# rocprofv3 --kernel-trace --stats summary", f"# command: {command}",
             f"# source_sha256 gemv: {source_hash('gemv')}",
             f"# source_sha256 gemm: {source_hash('gemm')}",
             f"{'kernel':90s} {'calls':>7s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{_short(r['Name']):90s} {int(r['Calls']):7d} {float(r['AverageNs'])/1e3:10.3f} "
                     f"{float(r['MinNs'])/1e3:10.3f} {float(r['MaxNs'])/1e3:10.3f} "
                     f"{float(r['Percentage']):6.2f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def committed_traffic(kind="gemv"):
    """HBM bytes per launch of awq_gemv (or awq_gemm, kind "gemm") from the
    committed counter summary, or None if there is none or the kernel's sources
    have changed since."""
    try:
        with open(TRAFFIC_SUMMARY if kind == "gemv" else GEMM_TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    sha = traffic = None
    for line in text.splitlines():
        if line.startswith("# source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif line.startswith("traffic_bytes_per_launch:"):
            traffic = float(line.split(":", 1)[1])
    if sha != source_hash(kind):
        return None
    return traffic


def config_line(cfg, r):
    """One configuration's figures: time per call and its fraction of the roofline
    that bounds it (HBM bytes for the GEMV entries, MFMA flops for the GEMMs)."""
    # The median of the line's replays where it has several (the headline's
    # own value is its first replay, the K timed calls).
    us = r["reps"]["median_us"] if "reps" in r else r["us_per_call"]
    line = {"config": cfg, "workload": r["workload"], "entry": r["entry"], "M": r["M"], "K": r["K"],
            "N": r["N"], "group_size": r["group_size"], "symmetric": r["symmetric"],
            "us_per_call": round(us, 3),
            "replays": r["reps"]["n"] if "reps" in r else r.get("replays", 1)}
    if "gbs" in r:
        gbs = r["alg_bytes"] / (us * 1e-6) / 1e9
        line.update(bound="hbm", gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4),
                    weight_copies=r["weight_copies"])
    else:
        flops = 2.0 * r["M"] * r["N"] * r["K"]
        b = alg_bytes(synth_workload(r["workload"]), r["M"])
        line.update(bound="mfma", tflops=round(r["tflops"], 1), frac=round(r["mfma_frac"], 4),
                    weight_copies=r["weight_copies"],
                    hbm_gbs=round(b / (r["us_per_call"] * 1e-6) / 1e9, 1),
                    hbm_frac=round(b / (r["us_per_call"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    arith_intensity=round(flops / b, 1))
    return line


def synth_workload(name):
    from w4a16_group_quantized_amd import synth
    return synth.WORKLOADS[name]


def main():
    global BENCH_LAYOUT
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--all", action="store_true", help="also time the other workloads")
    ap.add_argument("--layout", choices=sorted(LAYOUT), default=BENCH_LAYOUT,
                    help="qweight layout of the benchmarked layers")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--ceilings", action="store_true", help="only measure the two ceilings")
    ap.add_argument("--profile", choices=sorted(PROFILE_WORKLOAD), help="dispatch sequence for counter passes")
    ap.add_argument("--summarize-pmc", nargs="+", metavar=("OUT", "DIR"),
                    help="fold rocprofv3 --pmc CSV directories into a summary file")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("OUT", "DIR"),
                    help="fold a rocprofv3 --kernel-trace --stats directory into a summary file")
    ap.add_argument("--kind", choices=sorted(PROFILE_WORKLOAD), default="gemv", help="kernel of --summarize-pmc")
    ap.add_argument("--command", action="append", default=[],
                    help="command line(s) that produced the profiled data, recorded in the summary")
    args = ap.parse_args()
    BENCH_LAYOUT = args.layout
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1:], args.kind, args.command)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats[0], args.summarize_stats[1], " ; ".join(args.command))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards by output columns with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.profile:
        profile_run(args.profile)
        return
    if args.ceilings:
        print(json.dumps({"hbm_read": ceiling_read("decode_8b_gate"), "mfma_f16": ceiling_mfma()}))
        return
    from w4a16_group_quantized_amd import binding
    binding.load()

    head = bench_gemv("decode_8b_gate", args.steps, args.warmup, reps=5, hot=args.all)
    gemm = bench_gemm("prefill_out_proj", args.steps, args.warmup)
    # Every configuration of the workload list, each on its own entry point(s).
    configs = [
        ("cfg1", bench_gemv("tiny", args.steps, args.warmup, reps=CONFIG_REPS, max_copies=2)),
        ("cfg2", head),
        ("cfg3", bench_gemv("gate_up_m16", args.steps, args.warmup, reps=CONFIG_REPS)),
        ("cfg3", bench_gate_up("gate_up_m16", 16, args.steps, args.warmup)),
        ("cfg3", bench_gemm("gate_up_m16", args.steps, args.warmup, rotate=True)),
        ("cfg4", gemm),
        ("cfg5a", bench_gemv("sym70b_m1", args.steps, args.warmup, reps=CONFIG_REPS)),
        ("cfg5b", bench_gemm("sym70b_m4096", max(5, args.steps // 40), 2)),
    ]
    extra = []
    if args.all:
        extra.append(bench_gate_up("gate_up_m16", 1, args.steps, args.warmup))
        extra.append(bench_gemm_gate_up("gate_up_m16", 2048, 20, 3))
        for m in (64, 256, 512):
            extra.append(bench_gemm_splitk("prefill_out_proj", m, 100, 10))
        extra.append(bench_quantize("decode_8b_gate", 20, 3))
        extra.append(bench_scale_search("decode_8b_gate", 4096, 20, 3))
        extra.append(torch_matmul_context("sym70b_m4096", 5))

    traffic = committed_traffic()
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
                   "launch": "hip_graph", "layout": BENCH_LAYOUT},
        "roofline": {"bound": "hbm", "achieved": round(head["gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(head["hbm_frac"], 4), "traffic": traffic},
        "timing": {"replays": head["reps"]["n"], "calls_each": head["reps"]["calls_each"],
                   "median_us": round(head["reps"]["median_us"], 3),
                   "min_us": round(head["reps"]["min_us"], 3),
                   "max_us": round(head["reps"]["max_us"], 3)},
        "gemm": {"workload": gemm["workload"], "M": gemm["M"], "K": gemm["K"], "N": gemm["N"],
                 "tflops": round(gemm["tflops"], 1), "peak": MFMA_F16_PEAK_TFLOPS,
                 "frac": round(gemm["mfma_frac"], 4), "us_per_call": round(gemm["us_per_call"], 2)},
        # the metric's GEMM half: awq_gemm's kernel on the prefill shape against
        # the fp16 MFMA peak, in the same form as the decode kernel's roofline
        "roofline_gemm": {"bound": "mfma", "achieved": round(gemm["tflops"], 1),
                          "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(gemm["mfma_frac"], 4),
                          "traffic": committed_traffic("gemm")},
    }
    if "hot_cache_us" in head:
        out["timing"]["hot_cache_us"] = round(head["hot_cache_us"], 3)
    read, mfma = ceiling_read("decode_8b_gate"), ceiling_mfma()
    read70 = ceiling_read("sym70b_m1", steps=50)
    gemv70 = next(r for c, r in configs if c == "cfg5a")
    out["ceilings"] = {"hbm_read": read, "gemv_frac_of_read": round(head["gbs"] / read["gbs"], 4),
                       "hbm_read_sym70b_m1": read70,
                       "gemv_sym70b_m1_frac_of_read": round(gemv70["gbs"] / read70["gbs"], 4),
                       "mfma_f16": mfma, "gemm_frac_of_mfma": round(gemm["tflops"] / mfma["tflops"], 4)}
    out["configs"] = [config_line(cfg, r) for cfg, r in configs]
    out["context"] = {"torch_matmul": torch_matmul_context("prefill_out_proj", 50)}
    if extra:
        out["extra"] = extra
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
