"""The fused kernels inside a captured HIP graph, replayed: every replay gives
the eager results bit for bit.

The bench times the kernels as captured graphs, so their replays must be
exact.  One graph holds a decode GEMV, a fused gate/up GEMV, a prefill-shape
GEMM and a split-K GEMM with its caller-owned workspace (nothing is cleared
with a memset node: the split-K partials are fully overwritten each call).  It
is replayed three times, with other eager work and device synchronizations
between the replays, and the outputs are cleared before each replay so that a
replay that skipped a kernel would show.
"""
import numpy as np
import pytest
import torch

from gpu_cases import device_layer, workload_host
from parity import to_dev
from w4a16_group_quantized_amd import binding

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    dec = device_layer("decode_8b_gate")
    gu = device_layer("gate_up_m16")
    pre = device_layer("prefill_out_proj")
    x1 = to_dev(workload_host("decode_8b_gate")[0])
    x16 = to_dev(workload_host("gate_up_m16")[0])
    xp = to_dev(workload_host("prefill_out_proj")[0])
    xs = xp[:64].contiguous()
    splits = 4
    ws = torch.empty(binding.load().awq_gemm_splitk_workspace_bytes(64, pre.N, splits),
                     dtype=torch.uint8, device="cuda")
    outs = [torch.empty((1, dec.N), dtype=torch.float16, device="cuda"),
            torch.empty((16, gu.N // 2), dtype=torch.float16, device="cuda"),
            torch.empty((xp.shape[0], pre.N), dtype=torch.float16, device="cuda"),
            torch.empty((64, pre.N), dtype=torch.float16, device="cuda")]
    stream = torch.cuda.Stream()

    def calls():
        binding.gemv(x1, dec, out=outs[0], stream=stream)
        binding.gemv_gate_up(x16, gu, out=outs[1], stream=stream)
        binding.gemm(xp, pre, out=outs[2], stream=stream)
        binding.gemm_splitk(xs, pre, splits, out=outs[3], stream=stream, workspace=ws)

    with torch.cuda.stream(stream):
        calls()
    stream.synchronize()
    eager = [o.clone() for o in outs]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        calls()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        ws.fill_(0xFF)
        # unrelated eager work on the default stream between replays
        junk = binding.gemm(xs, pre)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}, output {i}"
        del junk
