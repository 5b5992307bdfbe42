"""GPU parity of the split-K GEMM (awq_gemm_splitk) against the oracle.

Each slice dequantizes exactly like awq_gemm and sums in fp32; the slices are
added in a fixed order and rounded once, so the output is held to the layer's
parity bar and repeated calls are bit-identical.  Cases cover 64-k and 32-k
steps, group indexing by shift and by division, one group per column, both
variants, ragged M and N, 64-row tiles (up to 64 rows) and 128-row ones, and
the automatic choice of slices.
"""
import numpy as np
import pytest
import torch

from gpu_cases import device_case, device_layer, oracle_case, random_case
from parity import assert_y_close, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding, synth

import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N,G,sym,splits", [
    (64, 4096, 512, 128, False, 4),      # 64-k steps, group by shift
    (37, 1024, 200, 128, False, 2),      # ragged M and N
    (1, 2048, 136, 2048, True, 8),       # one group per column
    (300, 2048, 264, 64, True, 4),       # several row tiles
    (130, 1536, 72, 96, False, 4),       # 32-k steps, group index by division
    (16, 8192, 64, 8192, False, 16),     # one group, 16 slices of 512 k
    (48, 1536, 72, 96, True, 4),         # 64-row tiles with 32-k steps, group by division
    (200, 2048, 264, 128, False, 4),     # 64-row tiles beyond 64 rows (4 x 2 tiles x 4 slices)
])
def test_splitk_parity(M, K, N, G, sym, splits):
    X, codes, zeros, scales = random_case(7000 + M + K + splits, M, K, N, G, sym)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    layer = device_case(codes, zeros, scales, G)
    y = to_host_bits(binding.gemm_splitk(to_dev(X), layer, splits))
    torch.cuda.synchronize()
    assert_y_close(y, Y16, f"splitk M={M} K={K} N={N} G={G} sym={sym} splits={splits}")


def test_splitk_auto_on_the_gate_up_shape():
    """M = 16 on the 4096 x 28672 layer: the automatic choice splits K, and
    sampled rows match the oracle."""
    w = synth.WORKLOADS["gate_up_m16"]
    X = synth.make_x(16, w.K, w.wid, w.n_outliers, w.outlier_gain)
    layer = device_layer("gate_up_m16")
    assert binding.splitk_splits(16, layer) > 1
    y = to_host_bits(binding.gemm_splitk(to_dev(X), layer))
    torch.cuda.synchronize()
    from gpu_cases import oracle_weight
    _, _, W = oracle_weight("gate_up_m16")
    rows = np.array([0, 5, 15])
    _, Y16 = oracle.load().matmul_w(np.ascontiguousarray(X[rows]), W)
    assert_y_close(y[rows], Y16, "splitk auto gate_up_m16")


def test_splitk_one_slice_is_gemm():
    X, codes, zeros, scales = random_case(11, 40, 1024, 136, 128, False)
    layer = device_case(codes, zeros, scales, 128)
    x = to_dev(X)
    a = to_host_bits(binding.gemm_splitk(x, layer, 1))
    b = to_host_bits(binding.gemm(x, layer))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)


def test_splitk_deterministic():
    X, codes, zeros, scales = random_case(12, 64, 2048, 256, 128, False)
    layer = device_case(codes, zeros, scales, 128)
    x = to_dev(X)
    runs = [to_host_bits(binding.gemm_splitk(x, layer, 8)) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(np.array_equal(runs[0], r) for r in runs[1:])
