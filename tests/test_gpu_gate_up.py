"""GPU parity of the fused gate/up entry (awq_gemv_gate_up) against the oracle.

The layer's N = 2I columns are [gate | up]; the oracle computes the layer's
fp64 sums and h = fp16(SiLU(gate) * up) from them (no intermediate rounding).
The kernel works from its fp32 sums with an fp32 SiLU, so h is held to the
same bar as Y.  Shapes cover the concatenated gate+up workload at its batch of
16 and at decode batches, the 70B symmetric layer, ragged column counts, and the
degenerate all-zero gate, where h is exactly zero.
"""
import numpy as np
import pytest
import torch

from gpu_cases import device_case, device_layer, oracle_weight, random_case, workload_host
from parity import assert_y_close, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding

import oracle

pytestmark = pytest.mark.gpu


def _oracle_h(X, W):
    Y64, _ = oracle.load().matmul_w(X, W)
    return oracle.load().gate_up(Y64)


@pytest.mark.parametrize("name,M", [("gate_up_m16", 16), ("gate_up_m16", 1), ("gate_up_m16", 4),
                                    ("sym70b_m1", 1), ("sym70b_m1", 8),
                                    ("sym70b_m1", 16)])   # X of 256 KB: staged segment by segment
def test_workload_gate_up(name, M):
    X, _, _, _ = workload_host(name)
    if X.shape[0] < M:                                  # more rows of the same distribution
        X = np.concatenate([X] * M, axis=0)[:M]
        X = np.ascontiguousarray(X)
    X = np.ascontiguousarray(X[:M])
    _, _, W = oracle_weight(name)
    h = to_host_bits(binding.gemv_gate_up(to_dev(X), device_layer(name)))
    torch.cuda.synchronize()
    assert_y_close(h, _oracle_h(X, W), f"gate_up {name} M={M}")


@pytest.mark.parametrize("M,K,I,G,sym", [
    (1, 128, 8, 128, False), (3, 256, 136, 128, False), (16, 1024, 40, 256, True),
    (5, 2048, 264, 128, False), (2, 384, 72, 384, True), (16, 4096, 520, 128, False),
    (11, 2048, 136, 256, True), (16, 1152, 136, 128, False), (1, 11008, 264, 128, True),
    (6, 1280, 40, 256, False), (3, 2688, 72, 128, False), (4, 1664, 40, 128, True),
    # X beyond LDS at one row (130 KB) and at four rows (224 KB): staged segment by segment
    (1, 66560, 8, 128, False), (4, 28672, 40, 128, True),
])
def test_ragged_gate_up(M, K, I, G, sym):
    X, codes, zeros, scales = random_case(900 + M + K, M, K, 2 * I, G, sym)
    o = oracle.load()
    W = o.dequant(o.pack(codes), scales, None if zeros is None else o.pack_zeros(zeros), G)
    h = to_host_bits(binding.gemv_gate_up(to_dev(X), device_case(codes, zeros, scales, G)))
    torch.cuda.synchronize()
    assert_y_close(h, _oracle_h(X, W), f"gate_up M={M} K={K} I={I} G={G} sym={sym}")


def test_zero_gate_gives_zero():
    """Gate codes equal to their zero points: every gate sum is 0 and h = 0.  The
    kernel recovers sum x (q - z) from fp32 sums of biased values, so its gate is
    zero up to their rounding; h stays within the bar of the up sums' scale."""
    M, K, I, G = 4, 512, 64, 128
    X, codes, zeros, scales = random_case(77, M, K, 2 * I, G, False)
    codes[:, :I] = 0
    zeros[:, :I] = 0
    o = oracle.load()
    W = o.dequant(o.pack(codes), scales, o.pack_zeros(zeros), G)
    Y64, _ = o.matmul_w(X, W)
    assert np.all(Y64[:, :I] == 0.0)
    assert np.all((o.gate_up(Y64) & 0x7FFF) == 0)
    h = to_host_bits(binding.gemv_gate_up(to_dev(X), device_case(codes, zeros, scales, G)))
    torch.cuda.synchronize()
    hv = h.view(np.float16).astype(np.float64)
    assert np.all(np.isfinite(hv))
    assert np.abs(hv).max() <= 1e-2 * np.abs(Y64[:, I:]).max()


def test_gate_up_equals_unfused_within_bar():
    """The fused entry and SiLU(gate) * up applied to the plain GEMV's fp16 Y agree
    within the parity bar (they differ only by Y's rounding to fp16)."""
    name = "gate_up_m16"
    X, _, _, _ = workload_host(name)
    layer = device_layer(name)
    x = to_dev(X)
    h = binding.gemv_gate_up(x, layer).float()
    y = binding.gemv(x, layer).float()
    I = layer.N // 2
    ref = torch.nn.functional.silu(y[:, :I]) * y[:, I:]
    torch.cuda.synchronize()
    err = (h - ref).abs().max().item()
    assert err <= 1e-2 * ref.abs().max().item(), err


def test_gate_up_empty_batch():
    layer = device_layer("gate_up_m16")
    x = torch.empty((0, layer.K), dtype=torch.float16, device="cuda")
    out = binding.gemv_gate_up(x, layer)
    assert tuple(out.shape) == (0, layer.N // 2)


# --- the batched entry: awq_gemm_gate_up -------------------------------------

def _sample(M, count, seed):
    if M <= count:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(1, M - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], rest]))


@pytest.mark.parametrize("name,M", [("gate_up_m16", 16), ("gate_up_m16", 300), ("gate_up_m16", 2048),
                                    ("sym70b_m1", 64)])
def test_gemm_gate_up_workload(name, M):
    from w4a16_group_quantized_amd import synth
    w = synth.WORKLOADS[name]
    X = synth.make_x(M, w.K, 1000 + M, w.n_outliers, w.outlier_gain)
    _, _, W = oracle_weight(name)
    h = to_host_bits(binding.gemm_gate_up(to_dev(X), device_layer(name)))
    torch.cuda.synchronize()
    rows = _sample(M, 24, M)
    assert_y_close(h[rows], _oracle_h(np.ascontiguousarray(X[rows]), W),
                   f"gemm gate_up {name} M={M} rows={len(rows)}")


@pytest.mark.parametrize("M,K,I,G,sym", [
    (37, 512, 200, 64, False), (130, 256, 8, 128, True), (1, 1024, 264, 256, False),
    (257, 768, 136, 768, True), (64, 1024, 136, 128, True), (65, 512, 72, 64, False),
])
def test_gemm_gate_up_ragged(M, K, I, G, sym):
    X, codes, zeros, scales = random_case(1300 + M + I, M, K, 2 * I, G, sym)
    o = oracle.load()
    W = o.dequant(o.pack(codes), scales, None if zeros is None else o.pack_zeros(zeros), G)
    h = to_host_bits(binding.gemm_gate_up(to_dev(X), device_case(codes, zeros, scales, G)))
    torch.cuda.synchronize()
    assert_y_close(h, _oracle_h(X, W), f"gemm gate_up M={M} K={K} I={I} G={G} sym={sym}")


def test_gemm_gate_up_onehot_saturated():
    """One-hot rows of X pick one dequantized weight row, so the gate and up sums
    are exactly w(k, n) and w(k, I + n) and h = fp16(SiLU(w_g) w_u) with an fp32
    SiLU; checked against the oracle's fp64 SiLU within the bar, and exactly 0
    where the gate weight is 0."""
    M, K, I, G = 64, 256, 64, 64
    X, codes, zeros, scales = random_case(4242, M, K, 2 * I, G, False)
    X = np.zeros((M, K), dtype=np.uint16)
    X[np.arange(M), np.arange(M) * 3 % K] = 0x3C00
    o = oracle.load()
    W = o.dequant(o.pack(codes), scales, o.pack_zeros(zeros), G)
    h = to_host_bits(binding.gemm_gate_up(to_dev(X), device_case(codes, zeros, scales, G)))
    torch.cuda.synchronize()
    ref = _oracle_h(X, W)
    assert_y_close(h, ref, "gemm gate_up one-hot")
    gate_zero = (W[np.arange(M) * 3 % K][:, :I] & 0x7FFF) == 0
    assert np.all((h[gate_zero] & 0x7FFF) == 0)
