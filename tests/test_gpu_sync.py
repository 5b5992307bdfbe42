"""The AWQ_SYNC debugging mode: with it set, every call waits for its stream
before returning (the stream is idle when the call returns) and the outputs are
those of the default mode bit for bit; a call made while its stream is being
captured into a graph still captures and replays (a capture cannot wait).

The library reads AWQ_SYNC once per process, so the AWQ_SYNC side runs in a
child process, alone on the GPU while it runs, and hands its outputs back
through a file.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from gpu_cases import device_layer, workload_host
from parity import to_dev
from w4a16_group_quantized_amd import binding

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def compute():
    """Outputs of a decode GEMV (both word layouts), a GEMM, a split-K GEMM
    and a graph replay of a GEMV, as uint16 arrays; and whether the stream was
    idle right after the GEMM returned."""
    dec = device_layer("decode_8b_gate")
    pre = device_layer("prefill_out_proj")
    x1 = to_dev(workload_host("decode_8b_gate")[0])
    xp = to_dev(workload_host("prefill_out_proj")[0])
    out = {}
    out["gemv"] = binding.gemv(x1, dec)
    out["gemv_il"] = binding.gemv(x1, binding.repack(dec, binding.LAYOUT_INTERLEAVED))
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    y = torch.empty((xp.shape[0], pre.N), dtype=torch.float16, device="cuda")
    binding.gemm(xp, pre, out=y)
    idle = stream.query()
    out["gemm"] = y
    out["splitk"] = binding.gemm_splitk(xp[:64].contiguous(), pre, splits=4)
    side = torch.cuda.Stream()
    g_out = torch.empty((1, dec.N), dtype=torch.float16, device="cuda")
    with torch.cuda.stream(side):
        binding.gemv(x1, dec, out=g_out)      # warm-up outside the capture
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        binding.gemv(x1, dec, out=g_out)
    replays = []
    for _ in range(2):
        g_out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replays.append(g_out.clone())
    out["graph0"], out["graph1"] = replays
    torch.cuda.synchronize()
    return {k: v.cpu().view(torch.int16).numpy() for k, v in out.items()}, idle


CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[2])
import numpy as np
import test_gpu_sync
outs, idle = test_gpu_sync.compute()
np.savez(sys.argv[3], idle=np.array(idle), **outs)
print("child done", flush=True)
"""


def test_sync_mode_matches_default(tmp_path):
    assert os.environ.get("AWQ_SYNC", "") in ("", "0"), "the parent must run in the default mode"
    path = str(tmp_path / "sync_outputs.npz")
    env = dict(os.environ, AWQ_SYNC="1")
    print("child process with AWQ_SYNC=1", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, HERE, ROOT, path], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    got = np.load(path)
    assert bool(got["idle"]), "AWQ_SYNC=1: the stream still had work when awq_gemm returned"
    want, _ = compute()
    for name, w in want.items():
        assert np.array_equal(got[name], w), f"{name}: AWQ_SYNC=1 output differs from the default mode"
    assert np.array_equal(want["graph0"], want["gemv"]) and np.array_equal(want["graph1"], want["gemv"])
