"""Where a call's time goes: the library's decode GEMV, small-batch GEMV and
prefill GEMM kernels, compiled with per-wave timestamps (``timeline.hip``),
run the way ``bench.py`` runs them (a captured graph of back-to-back calls on
cold weight copies), with the stamps of the last call read back.

    python -m probes timeline [--out FILE]

Times are microseconds after the first wave of the call started; the stamps
come from the GPU's constant 100 MHz counter, the clocks from the shader clock
counter over the same interval.  The per-call time is the graph's, by events.
"""
from __future__ import annotations

import ctypes
import math
import os
import statistics as st
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TICK_US = 0.01   # s_memrealtime runs at 100 MHz


def _lib():
    from probes import LIBRARY
    if not os.path.exists(LIBRARY):
        raise RuntimeError(f"{LIBRARY} is missing: run probes.build() first")
    lib = ctypes.CDLL(LIBRARY)
    lib.awq_timeline_gemv.restype = ctypes.c_int
    lib.awq_timeline_gemv.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + \
        [ctypes.c_void_p]
    lib.awq_timeline_gemm.restype = ctypes.c_int
    lib.awq_timeline_gemm.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    lib.awq_timeline_read.restype = ctypes.c_int
    lib.awq_timeline_read.argtypes = [ctypes.c_void_p]
    lib.awq_timeline_slots.restype = ctypes.c_int
    return lib


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _graph_time(call, layers, steps, reps, settle_s):
    """Per-call microseconds of a captured graph of ``steps`` calls cycling
    through ``layers`` (median of ``reps`` replays), after ``settle_s`` seconds
    of untimed replays; the last replay's last call leaves its stamps."""
    import torch
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(20):
            call(layers[i % len(layers)], stream)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            call(layers[i % len(layers)], stream)
    with torch.cuda.stream(stream):
        graph.replay()
    stream.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / steps)
    return st.median(ts)


def _stamps(lib, slots):
    n = lib.awq_timeline_slots()
    buf = (ctypes.c_ulonglong * (6 * n))()
    rc = lib.awq_timeline_read(buf)
    if rc != 0:
        raise RuntimeError(f"awq_timeline_read: hip error {rc}")
    return [[buf[f * n + s] for s in slots] for f in range(6)]


def _q(values):
    return f"median {st.median(values):.2f}, max {max(values):.2f}"


def gemv_timeline(name, kind, rows=None):
    """Timeline of awq_gemv's kernel ``kind`` (0 decode, 1 small batch) on a
    workload; returns the summary lines."""
    import dataclasses
    import torch
    import bench
    from w4a16_group_quantized_amd import binding, synth
    lib = _lib()
    w = synth.WORKLOADS[name]
    if rows is not None:
        w = dataclasses.replace(w, M=rows)
    bench.BENCH_LAYOUT = "blocked"
    copies = max(2, math.ceil(bench.ROTATE_BYTES / bench.alg_bytes(w, 0)))
    layers = bench.build_layers(w, copies)
    x = bench.to_dev(synth.make_x(w.M, w.K, w.wid, w.n_outliers, w.outlier_gain))
    y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")

    def call(lay, stream):
        rc = lib.awq_timeline_gemv(kind, x.data_ptr(), lay.qweight.data_ptr(), lay.scales.data_ptr(),
                                   _ptr(lay.qzeros), y.data_ptr(), w.M, w.K, w.N, w.G,
                                   stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"awq_timeline_gemv: hip error {rc}")

    ref = binding.gemv(x, layers[0])
    s = torch.cuda.Stream()
    call(layers[0], s)
    s.synchronize()
    same = bool(torch.equal(y, ref))
    per_call = _graph_time(call, layers, 200, 5, 0.0)
    strip = 16 * (4 if kind == 0 else 8)
    nwg, nw = (w.N + strip - 1) // strip, 8
    slots = [g * nw + v for g in range(nwg) for v in range(nw)]
    start, loop, red, end, c0, c1 = _stamps(lib, slots)
    t0 = min(start)
    rel = lambda a: [(v - t0) * TICK_US for v in a]
    loop_end = rel(loop)
    old = [loop_end[g * nw + v] for g in range(nwg) for v in range(nw // 2)]
    young = [loop_end[g * nw + v] for g in range(nwg) for v in range(nw // 2, nw)]
    wg_end = [max(loop_end[g * nw:(g + 1) * nw]) for g in range(nwg)]
    epi = [(end[i] - red[i]) * TICK_US for i in range(len(slots))]
    span = max(rel(end))
    clock = st.median((c1[i] - c0[i]) / ((loop[i] - start[i]) * TICK_US * 1e3)
                      for i in range(len(slots)) if loop[i] > start[i])
    return [
        f"## awq_gemv on {name}: M={w.M} K={w.K} N={w.N} G={w.G}, blocked words, "
        f"{nwg} workgroups x {nw} waves, {copies} cold weight copies",
        f"outputs equal to the library's awq_gemv: {same}",
        f"per call (graph of 200, median of 5 replays): {per_call:.2f} us",
        f"wave starts: {_q(rel(start))} us",
        f"segment loop ends, waves 0-{nw // 2 - 1}: {_q(old)} us",
        f"segment loop ends, waves {nw // 2}-{nw - 1}: {_q(young)} us",
        f"a workgroup's last loop end: {_q(wg_end)} us",
        f"reduction, store and store completion (duration): {_q(epi)} us",
        f"first wave start to last wave end: {span:.2f} us; outside every wave: "
        f"{per_call - span:.2f} us per call",
        f"shader clock over the loop: {clock:.3f} GHz (median over waves)",
    ]


def gemm_timeline(name="prefill_out_proj"):
    """Timeline of awq_gemm's fast path on a workload; returns the summary lines."""
    import torch
    import bench
    from w4a16_group_quantized_amd import binding, synth
    lib = _lib()
    w = synth.WORKLOADS[name]
    bench.BENCH_LAYOUT = "blocked"
    layers = bench.build_layers(w, 1)
    x = bench.to_dev(synth.make_x(w.M, w.K, w.wid, w.n_outliers, w.outlier_gain))
    y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")

    def call(lay, stream):
        rc = lib.awq_timeline_gemm(x.data_ptr(), lay.qweight.data_ptr(), lay.scales.data_ptr(),
                                   _ptr(lay.qzeros), y.data_ptr(), w.M, w.K, w.N, w.G,
                                   stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"awq_timeline_gemm: hip error {rc}")

    ref = binding.gemm(x, layers[0])
    s = torch.cuda.Stream()
    call(layers[0], s)
    s.synchronize()
    same = bool(torch.equal(y, ref))
    per_call = _graph_time(call, layers, 100, 5, 0.1)
    bm = 256 if (w.M + 255) // 256 * ((w.N + 255) // 256) >= 512 else 128
    nwg = ((w.M + bm - 1) // bm) * ((w.N + 255) // 256)
    start, loop0, loop1, end, c0, c1 = _stamps(lib, list(range(nwg)))
    t0 = min(start)
    pro = [(loop0[i] - start[i]) * TICK_US for i in range(nwg)]
    loop = [(loop1[i] - loop0[i]) * TICK_US for i in range(nwg)]
    epi = [(end[i] - loop1[i]) * TICK_US for i in range(nwg)]
    span = (max(end) - t0) * TICK_US
    clock = [(c1[i] - c0[i]) / ((loop1[i] - loop0[i]) * TICK_US * 1e3) for i in range(nwg)]
    steps = w.K // 64
    busy = 32 * 32 * steps   # 32 MFMAs of 32 busy cycles per wave and 64-k step (128-row tiles)
    return [
        f"## awq_gemm on {name}: M={w.M} K={w.K} N={w.N} G={w.G}, blocked words, "
        f"{nwg} workgroups",
        f"outputs equal to the library's awq_gemm: {same}",
        f"per call (graph of 100 after 0.1 s of settling replays, median of 5): {per_call:.2f} us",
        f"workgroup starts spread over: {(max(start) - t0) * TICK_US:.2f} us",
        f"prologue (first loads landed): {_q(pro)} us",
        f"K loop: {_q(loop)}, min {min(loop):.2f} us",
        f"epilogue (tile stored, stores completed): {_q(epi)} us",
        f"first start to last end: {span:.2f} us; outside every wave: {per_call - span:.2f} us per call",
        f"shader clock over the K loop: median {st.median(clock):.3f} GHz "
        f"(min {min(clock):.3f}, max {max(clock):.3f})",
        f"matrix cores busy over the K loop (128-row tiles: {busy} MFMA cycles per SIMD): "
        f"{busy / (st.median(loop) * 1e3 * st.median(clock)):.3f}" if bm == 128 else "",
    ]


def main(out=None):
    import torch
    torch.cuda.set_device(0)
    lines = ["# timeline probe (per-wave timestamps in the library's kernels, probes/timeline.hip)",
             f"# command: python -m probes timeline --out {out or '<file>'}   (repo root, after build())",
             ""]
    for block in (gemv_timeline("decode_8b_gate", 0), gemv_timeline("gate_up_m16", 1),
                  gemm_timeline("prefill_out_proj")):
        lines += [ln for ln in block if ln] + [""]
        print("\n".join(block), flush=True)
    if out:
        with open(out, "w") as f:
            f.write("\n".join(lines))
