"""GPU parity of the fused layer (awq_gemv, awq_gemm) against the oracle.

Y is compared with the oracle's fp16 result under the bar in ``parity``; the
one-hot and identity cases, where exactly one product reaches each output, are
compared bit for bit with the oracle's dequantized weight.  Full-size workloads
run in the launch configuration the benchmark times; for the two large-batch
GEMMs the oracle computes a seeded sample of rows (all columns), since every
output row depends on its own row of X only.
"""
import os

import numpy as np
import pytest
import torch

from gpu_cases import (device_case, device_layer, oracle_case, oracle_weight, random_case,
                       workload_host)
from parity import assert_y_close, same_halves_up_to_zero_sign, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding, synth

import oracle

pytestmark = pytest.mark.gpu

ENTRY = {"gemv": binding.gemv, "gemm": binding.gemm}
HOST_THREADS = min(16, len(os.sched_getaffinity(0)))


def _sample_rows(M, count, seed):
    if M <= count:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(1, M - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], rest]))


def _leading_and_seeded_rows(M, lead, count, seed):
    """The first ``lead`` rows, the last one, and ``count`` seeded others."""
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(lead, M - 1), size=count, replace=False)
    return np.unique(np.concatenate([np.arange(lead), [M - 1], rest]))


@pytest.mark.parametrize("entry,name", [
    ("gemv", "tiny"), ("gemv", "decode_8b_gate"), ("gemv", "gate_up_m16"), ("gemv", "sym70b_m1"),
    ("gemm", "tiny"), ("gemm", "gate_up_m16"), ("gemm", "prefill_out_proj"),
    ("gemm", "sym70b_m4096"),
])
def test_workload_parity(entry, name):
    w = synth.WORKLOADS[name]
    X, _, _, _ = workload_host(name)
    _, _, W = oracle_weight(name)
    layer = device_layer(name)
    y = to_host_bits(ENTRY[entry](to_dev(X), layer))
    torch.cuda.synchronize()
    if w.M > 128 and w.K * w.N > 1 << 25:
        # the 70B-shape batch: 64 leading rows, the last and 64 seeded ones (rows are independent)
        rows = _leading_and_seeded_rows(w.M, 64, 64, w.wid)
    else:
        rows = _sample_rows(w.M, 64, w.wid)
    _, Y16 = oracle.load().matmul_w_columns(np.ascontiguousarray(X[rows]), W, HOST_THREADS)
    assert_y_close(y[rows], Y16, f"{entry} {name} rows={len(rows)}")


RAGGED = [
    # M, K, N, G, symmetric
    (1, 8, 8, 8, False), (1, 32, 8, 32, True), (3, 136, 200, 8, False), (5, 256, 72, 64, False),
    (16, 512, 24, 512, True), (7, 1024, 264, 128, False), (2, 96, 40, 32, False),
    (1, 520, 8, 8, True), (16, 4096, 136, 128, False), (9, 192, 64, 96, False),
    (4, 1152, 520, 1152, True),
    # beyond four rows the decode kernel stages X segment by segment, 2, 3 or 4
    # chunks per lane: 7, 12 and 13 rows, with groups of one segment, of two, and
    # one group per column
    (12, 2048, 264, 128, False), (7, 4096, 200, 256, True), (13, 1024, 72, 1024, False),
    # up to four rows with X beyond LDS (172 and 164 KB): staged segment by segment too
    (3, 28672, 264, 128, False), (4, 20480, 1032, 256, True),
]


@pytest.mark.parametrize("entry", ["gemv", "gemm"])
@pytest.mark.parametrize("M,K,N,G,sym", RAGGED)
def test_ragged_parity(entry, M, K, N, G, sym):
    seed = 1000 + M * 7 + K * 3 + N + G
    X, codes, zeros, scales = random_case(seed, M, K, N, G, sym)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    layer = device_case(codes, zeros, scales, G)
    y = to_host_bits(ENTRY[entry](to_dev(X), layer))
    assert_y_close(y, Y16, f"{entry} M={M} K={K} N={N} G={G} sym={sym}")


@pytest.mark.parametrize("M,K,N,G", [(37, 200, 136, 8), (130, 1032, 264, 8), (257, 1024, 8, 128),
                                     (300, 4096, 520, 128),
                                     # 32-k steps: G a multiple of 32, K of 128 but not 256
                                     (130, 640, 264, 32), (300, 384, 520, 128), (65, 896, 136, 64),
                                     # 64-row tiles (up to 64 rows), 32-k and 64-k steps
                                     (64, 640, 264, 32), (50, 2048, 200, 128)])
def test_gemm_large_ragged(M, K, N, G):
    X, codes, zeros, scales = random_case(77 + M, M, K, N, G, False)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    layer = device_case(codes, zeros, scales, G)
    assert_y_close(to_host_bits(binding.gemm(to_dev(X), layer)), Y16, f"gemm M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,G,sym", [
    (2200, 384, 14584, 128, False),    # 256-row tiles (>= 512 of them), ragged M and N
    (2304, 384, 14592, 96, True),      # group of 3 steps: index by division
    (2200, 512, 14584, 512, False),    # one group per column
])
def test_gemm_wide_tiles(M, K, N, G, sym):
    """Shapes large enough for the 256-row-tile path, checked on sampled rows."""
    X, codes, zeros, scales = random_case(5000 + M + G, M, K, N, G, sym)
    rows = _sample_rows(M, 16, M + N)
    _, Y16 = oracle_case(X, codes, zeros, scales, G, rows=rows)
    y = to_host_bits(binding.gemm(to_dev(X), device_case(codes, zeros, scales, G)))
    torch.cuda.synchronize()
    assert_y_close(y[rows], Y16, f"gemm wide M={M} K={K} N={N} G={G} sym={sym}")


@pytest.mark.parametrize("entry", ["gemv", "gemm"])
@pytest.mark.parametrize("K,N,G,sym", [(512, 512, 128, False), (256, 200, 8, False),
                                       (1024, 136, 1024, True), (1024, 136, 1024, False)])
def test_onehot_rows_bit_exact(entry, K, N, G, sym):
    """X row m = e_k(m): each output is one exact product, rounded once.  On
    one-group layers the GEMM multiplies the sum q - z by the scale after the
    matrix cores: with x = 1 that product is still exact in fp32, so the output
    is still the dequantized weight bit for bit."""
    _, codes, zeros, scales = random_case(5 + K, 1, K, N, G, sym)
    W, _ = oracle_case(np.zeros((1, K), np.uint16), codes, zeros, scales, G)
    ks = np.random.default_rng(K + N).choice(K, size=16, replace=False)
    X = np.zeros((16, K), dtype=np.uint16)
    X[np.arange(16), ks] = 0x3C00
    layer = device_case(codes, zeros, scales, G)
    y = to_host_bits(ENTRY[entry](to_dev(X), layer))
    assert same_halves_up_to_zero_sign(y, W[ks])


@pytest.mark.parametrize("K,N,G", [(256, 136, 64), (256, 136, 256)])
def test_gemm_identity_returns_weight(K, N, G):
    """X = I_K through awq_gemm gives the whole dequantized matrix (also with one
    group per column, where the scale multiplies the fp32 sum)."""
    _, codes, zeros, scales = random_case(42, 1, K, N, G, False)
    W, _ = oracle_case(np.zeros((1, K), np.uint16), codes, zeros, scales, G)
    X = np.zeros((K, K), dtype=np.uint16)
    X[np.arange(K), np.arange(K)] = 0x3C00
    y = to_host_bits(binding.gemm(to_dev(X), device_case(codes, zeros, scales, G)))
    assert same_halves_up_to_zero_sign(y, W)


@pytest.mark.parametrize("entry,name", [("gemv", "decode_8b_gate"), ("gemv", "gate_up_m16"),
                                        ("gemm", "prefill_out_proj")])
def test_deterministic_and_power_of_two(entry, name):
    """Two runs are bit-identical, and doubling X doubles Y bit for bit.

    The decode kernel stages odd k of X as x/16; below |x| = 2^-10 that value is
    an fp16 subnormal whose rounding does not commute with doubling, so such
    entries are zeroed first (they move Y by far less than the tolerance)."""
    X, _, _, _ = workload_host(name)
    X = X.copy()
    X[np.abs(X.view(np.float16).astype(np.float64)) < 2.0 ** -9] = 0
    layer = device_layer(name)
    xd = to_dev(X)
    y1 = ENTRY[entry](xd, layer)
    y2 = ENTRY[entry](xd, layer)
    y3 = ENTRY[entry](xd * 2, layer)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # fp16 rounding commutes with doubling except where the doubled value is
    # still subnormal in fp16 (|Y| below 2^-14), so those outputs are skipped
    normal = y1.float().abs() >= 2.0 ** -13
    assert torch.equal((y1.float() * 2).half()[normal].view(torch.int16), y3[normal].view(torch.int16))


@pytest.mark.parametrize("M,K,N,G", [(1, 4096, 4096, 128), (16, 4096, 4096, 128),
                                     (1, 14336, 4096, 128), (8, 4096, 8192, 128),
                                     (16, 14336, 4096, 128)])   # X beyond LDS: staged per segment
def test_gemv_narrow_layers(M, K, N, G):
    """Layers whose 64-column strips would leave half the CUs idle (attention
    output and down projections of the 8B model) run on 32-column strips."""
    X, codes, zeros, scales = random_case(5100 + M + K + N, M, K, N, G, False)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    y = to_host_bits(binding.gemv(to_dev(X), device_case(codes, zeros, scales, G)))
    assert_y_close(y, Y16, f"gemv M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,G,sym", [
    (1, 11008, 4096, 128, False), (4, 11008, 4096, 128, True), (16, 11008, 4096, 128, False),
    (1, 13824, 5120, 128, True), (1, 11264, 4096, 128, False), (3, 1152, 200, 128, False),
    (7, 2176, 264, 128, True), (16, 1280, 136, 256, False), (2, 1536, 72, 384, True),
])
def test_gemv_uneven_k(M, K, N, G, sym):
    """K whose 128-k segments do not split evenly over the eight waves of a
    workgroup (K = 11008: 86 segments; 11264: 88, eleven a wave, odd against a
    two-deep pipeline): the first waves take one segment more.  Groups of 256
    and 384 put wave boundaries inside a group."""
    X, codes, zeros, scales = random_case(5300 + M + K + N, M, K, N, G, sym)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    y = to_host_bits(binding.gemv(to_dev(X), device_case(codes, zeros, scales, G)))
    assert_y_close(y, Y16, f"gemv M={M} K={K} N={N} G={G} sym={sym}")


SCALE_CASES = [(1, 4096, 264, 128, False), (16, 1024, 136, 128, True), (5, 2048, 200, 2048, False)]


@pytest.mark.parametrize("entry,M,K,N,G,sym",
                         [("gemv",) + c for c in SCALE_CASES] +
                         [("gemm",) + c for c in SCALE_CASES + [(300, 1024, 264, 1024, True)]])
def test_doubling_scales_doubles_y(entry, M, K, N, G, sym):
    """Every scale times 2 (exponent + 1, exact) doubles Y bit for bit: in the
    exact dequantization fp16(2 s (q - z)) = 2 fp16(s (q - z)), in the folded
    decode path and in the one-group GEMM the scale multiplies an fp32 sum, and
    fp32 and fp16 rounding commute with doubling away from the subnormals."""
    X, codes, zeros, scales = random_case(4400 + M + K + G, M, K, N, G, sym)
    X = X.copy()
    X[np.abs(X.view(np.float16).astype(np.float64)) < 2.0 ** -9] = 0   # see the test above
    xd = to_dev(X)
    y1 = ENTRY[entry](xd, device_case(codes, zeros, scales, G))
    y2 = ENTRY[entry](xd, device_case(codes, zeros, (scales + 0x0400).astype(np.uint16), G))
    torch.cuda.synchronize()
    normal = y1.float().abs() >= 2.0 ** -13
    assert normal.float().mean().item() > 0.99
    assert torch.equal((y1.float() * 2).half()[normal].view(torch.int16), y2[normal].view(torch.int16))


def test_gemv_equals_gemm_on_decode_shape():
    """Both entry points compute the same layer (within the bar of each other)."""
    X, _, _, _ = workload_host("gate_up_m16")
    layer = device_layer("gate_up_m16")
    a = to_host_bits(binding.gemv(to_dev(X), layer))
    b = to_host_bits(binding.gemm(to_dev(X), layer))
    assert_y_close(a, b, "gemv vs gemm")


@pytest.mark.parametrize("entry", ["gemv", "gemm"])
def test_empty_batch(entry):
    layer = device_layer("tiny")
    x = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    y = ENTRY[entry](x, layer)
    assert y.shape == (0, 512)


def test_gemv_rejects_batches_above_16():
    layer = device_layer("tiny")
    x = torch.zeros((17, 512), dtype=torch.float16, device="cuda")
    with pytest.raises(binding.AwqError) as e:
        binding.gemv(x, layer)
    assert e.value.status == 4


def test_misaligned_pointer_is_rejected():
    layer = device_layer("tiny")
    buf = torch.zeros(512 + 8, dtype=torch.float16, device="cuda")
    x = buf[1:513].view(1, 512)            # 2 bytes past a 16-byte boundary
    with pytest.raises(binding.AwqError) as e:
        binding.gemv(x, layer)
    assert e.value.status == 3


@pytest.mark.parametrize("M,K,N,G,sym", [
    (37, 768, 200, 768, False), (130, 256, 72, 256, False), (64, 2048, 136, 2048, True),
    (1, 1024, 264, 1024, False),
])
def test_gemm_one_group(M, K, N, G, sym):
    """One group per column (G == K): scales and zero points are loaded once per
    lane, past the last column included (ragged N); the matrix cores take q - z
    and each column's scale multiplies its fp32 sum, so Y is held to the layer's
    parity bar like the folded decode path."""
    X, codes, zeros, scales = random_case(9000 + M + K, M, K, N, G, sym)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    y = to_host_bits(binding.gemm(to_dev(X), device_case(codes, zeros, scales, G)))
    torch.cuda.synchronize()
    assert_y_close(y, Y16, f"gemm one group M={M} K={K} N={N} sym={sym}")


@pytest.mark.parametrize("M,K,N,G,sym,layout", [
    # Wide layers (128 columns per workgroup keep three quarters of the CUs busy) from three
    # rows up: paired strips, 64 columns of each half.  N / 2 not a multiple of 64 leaves a
    # ragged last strip in each half (canonical and interleaved words); blocked words need
    # N % 128 == 0.  An odd segment count per wave (K = 1280) takes the guarded pipeline.
    (3, 1024, 24592, 128, False, binding.LAYOUT_CANONICAL),
    (5, 1024, 24592, 256, True, binding.LAYOUT_INTERLEAVED),
    (8, 3072, 24592, 1024, True, binding.LAYOUT_CANONICAL),
    (12, 1280, 24592, 128, False, binding.LAYOUT_CANONICAL),
    (16, 2048, 24592, 128, False, binding.LAYOUT_INTERLEAVED),
    (16, 1024, 24704, 128, False, binding.LAYOUT_BLOCKED),
])
def test_paired_strips_parity(M, K, N, G, sym, layout):
    X, codes, zeros, scales = random_case(3100 + M + K + G, M, K, N, G, sym)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    layer = device_case(codes, zeros, scales, G)
    if layout != binding.LAYOUT_CANONICAL:
        layer = binding.repack(layer, layout)
    y = to_host_bits(binding.gemv(to_dev(X), layer))
    torch.cuda.synchronize()
    assert_y_close(y, Y16, f"gemv paired M={M} K={K} N={N} G={G} sym={sym} layout={layout}")
