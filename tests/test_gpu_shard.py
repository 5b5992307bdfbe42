"""Column slicing: the layer computed on column shards equals the full layer.

A shard [n0, n1) of a layer is qweight[:, n0:n1], scales[:, n0:n1] and
qzeros[:, n0/8:n1/8] (n0, n1 multiples of 8): each output column depends only
on its own packed column, scale and zero point.  This is how the layer would be
split over several GPUs (by output columns, no exchange), shown here on one GPU
through the C ABI.  awq_gemm sums every output column in an order that does not
depend on N, so its shards match the full call bit for bit; awq_gemv picks its
pipeline from the shape, so its shards are held to the parity bar against the
oracle instead.
"""
import numpy as np
import pytest
import torch

from gpu_cases import device_layer, oracle_weight, workload_host
from parity import assert_y_close, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding, synth

import oracle

pytestmark = pytest.mark.gpu


def _shard(layer: binding.Layer, n0: int, n1: int) -> binding.Layer:
    assert n0 % 8 == 0 and n1 % 8 == 0 and 0 <= n0 < n1 <= layer.N
    qz = None if layer.qzeros is None else layer.qzeros[:, n0 // 8:n1 // 8].contiguous()
    return binding.Layer(layer.qweight[:, n0:n1].contiguous(), layer.scales[:, n0:n1].contiguous(),
                         qz, layer.K, n1 - n0, layer.group_size)


def _bounds(N, cuts):
    return [0, *cuts, N]


@pytest.mark.parametrize("name,cuts", [
    ("prefill_out_proj", [1024, 2048, 3072]),          # four even shards
    ("gate_up_m16", [1000, 9000, 20000]),              # uneven shards, ragged tiles
    ("sym70b_m1", [3584 * i for i in range(1, 8)]),     # eight shards of the 70B layer
])
def test_gemm_shards_bit_identical(name, cuts):
    w = synth.WORKLOADS[name]
    X, _, _, _ = workload_host(name)
    x = to_dev(X)
    layer = device_layer(name)
    full = to_host_bits(binding.gemm(x, layer))
    b = _bounds(w.N, cuts)
    for n0, n1 in zip(b[:-1], b[1:]):
        part = to_host_bits(binding.gemm(x, _shard(layer, n0, n1)))
        torch.cuda.synchronize()
        assert np.array_equal(part, full[:, n0:n1]), f"{name} shard [{n0}, {n1})"


@pytest.mark.parametrize("name,cuts", [
    ("decode_8b_gate", [3584, 7168, 10752]),
    ("gate_up_m16", [1000, 9000, 20000]),
    ("sym70b_m1", [3584 * i for i in range(1, 8)]),
])
def test_gemv_shards_match_oracle(name, cuts):
    w = synth.WORKLOADS[name]
    X, _, _, _ = workload_host(name)
    _, _, W = oracle_weight(name)
    _, Y16 = oracle.load().matmul_w(X, W)
    x = to_dev(X)
    layer = device_layer(name)
    b = _bounds(w.N, cuts)
    parts = [to_host_bits(binding.gemv(x, _shard(layer, n0, n1))) for n0, n1 in zip(b[:-1], b[1:])]
    torch.cuda.synchronize()
    assert_y_close(np.concatenate(parts, axis=1), Y16, f"gemv {name} in {len(parts)} shards")
