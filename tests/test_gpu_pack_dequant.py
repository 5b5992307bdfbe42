"""GPU parity: packing and exact dequantization, bit for bit against the oracle."""
import numpy as np
import pytest

import oracle
from gpu_cases import device_layer, oracle_weight, workload_host
from parity import to_dev, to_host_bits
from w4a16_group_quantized_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,N", [(8, 8), (64, 24), (512, 512), (136, 200), (4096, 14336)])
def test_pack_matches_oracle(K, N):
    rng = np.random.default_rng(K * 7919 + N)
    codes = rng.integers(0, 256, (K, N), dtype=np.uint8)    # high bits must be ignored
    got = binding.pack(to_dev(codes)).cpu().numpy()
    assert np.array_equal(got, oracle.load().pack(codes))


@pytest.mark.parametrize("groups,N", [(1, 8), (4, 512), (3, 200), (32, 28672)])
def test_pack_zeros_matches_oracle(groups, N):
    rng = np.random.default_rng(groups * 31 + N)
    zeros = rng.integers(0, 256, (groups, N), dtype=np.uint8)
    got = binding.pack_zeros(to_dev(zeros)).cpu().numpy()
    assert np.array_equal(got, oracle.load().pack_zeros(zeros))


def _exhaustive_layer():
    """Every code, zero point and finite fp16 scale (the oracle's exhaustive pin
    layout): group g has zero g, row k has code k % 16, column n the n-th finite
    fp16 pattern as its scale."""
    all_h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = all_h[(all_h & 0x7C00) != 0x7C00]
    N, G, groups = finite.size, 16, 16
    K = G * groups
    codes = np.tile((np.arange(K) % 16).astype(np.uint8)[:, None], (1, N))
    zeros = np.tile(np.arange(groups, dtype=np.uint8)[:, None], (1, N))
    scales = np.ascontiguousarray(np.tile(finite[None, :], (groups, 1)))
    return codes, zeros, scales, G


def test_dequant_exhaustive_bit_exact():
    codes, zeros, scales, G = _exhaustive_layer()
    o = oracle.load()
    want = o.dequant(o.pack(codes), scales, o.pack_zeros(zeros), G)
    layer = binding.make_layer(to_dev(codes), to_dev(zeros), to_dev(scales), G)
    got = to_host_bits(binding.dequant(layer))
    assert np.array_equal(got, want), int(np.sum(got != want))
    # symmetric: no zero tensor, zero point 8
    want_s = o.dequant(o.pack(codes[:16]), scales[:1], None, 16)
    layer_s = binding.make_layer(to_dev(codes[:16]), None, to_dev(scales[:1]), 16)
    assert np.array_equal(to_host_bits(binding.dequant(layer_s)), want_s)


@pytest.mark.parametrize("name", ["tiny", "decode_8b_gate", "sym70b_m1"])
def test_dequant_workloads_bit_exact(name):
    Q, QZ, W = oracle_weight(name)
    layer = device_layer(name)
    assert np.array_equal(layer.qweight.cpu().numpy(), Q)
    if QZ is not None:
        assert np.array_equal(layer.qzeros.cpu().numpy(), QZ)
    got = to_host_bits(binding.dequant(layer))
    assert np.array_equal(got, W)


@pytest.mark.parametrize("K,N,G,sym", [(8, 8, 8, False), (24, 16, 8, True), (136, 200, 8, False),
                                       (256, 72, 64, False), (512, 24, 512, True)])
def test_dequant_ragged_bit_exact(K, N, G, sym):
    codes, zeros, scales = synth.make_layer(K, N, G, sym, 0.001, 0.05, K + N + G)
    o = oracle.load()
    want = o.dequant(o.pack(codes), scales, None if sym else o.pack_zeros(zeros), G)
    layer = binding.make_layer(to_dev(codes), None if sym else to_dev(zeros), to_dev(scales), G)
    assert np.array_equal(to_host_bits(binding.dequant(layer)), want)
