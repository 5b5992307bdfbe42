"""GPU parity of the group quantizer (awq_quantize) against the oracle.

Codes and zero points are integers decided in fp32 on both sides, and each
scale is the exact (hi - lo) / 15 or max|w| / 7 rounded once to fp16, so all
three are compared bit for bit.  Shapes cover several
group sizes (including one group per column), ragged column counts, both
variants, weights spanning many magnitudes, constant and all-zero groups, and
a Llama-shaped layer; the quantized layer then runs through the fused GEMV
and is checked against the oracle's layer built from the same codes.
"""
import numpy as np
import pytest
import torch

from parity import assert_y_close, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding, synth

import oracle

pytestmark = pytest.mark.gpu


def _weights(seed, K, N, spread=True):
    """fp16 weights ~ N(0, sigma_n) with per-column sigma spanning 1e-3 .. 1 (seeded)."""
    rng = np.random.default_rng(seed)
    sigma = np.exp(rng.uniform(np.log(1e-3), 0.0, (1, N))) if spread else 0.02
    return (rng.standard_normal((K, N)) * sigma).astype(np.float16).view(np.uint16)


def _check(W, G, sym, what):
    o = oracle.load()
    codes, S, Z = o.quantize(W, G, sym)
    lay = binding.quantize(to_dev(W), G, sym)
    torch.cuda.synchronize()
    assert np.array_equal(lay.qweight.cpu().numpy(), o.pack(codes)), f"{what}: codes"
    assert np.array_equal(to_host_bits(lay.scales), S), f"{what}: scales"
    if sym:
        assert lay.qzeros is None
    else:
        assert np.array_equal(lay.qzeros.cpu().numpy(), o.pack_zeros(Z)), f"{what}: zeros"
    return codes, S, Z, lay


@pytest.mark.parametrize("K,N,G,sym", [
    (128, 64, 128, False), (256, 40, 64, False), (512, 136, 128, True), (64, 8, 8, False),
    (1024, 200, 1024, True), (384, 24, 32, False), (4096, 512, 128, False), (96, 72, 96, True),
    (2048, 136, 2048, False), (8192, 72, 8192, True), (3072, 64, 1536, False),
    # long groups over several 64-column tiles: 16 waves a group (4096), 8 (1024)
    (4096, 1032, 4096, False), (2048, 520, 1024, True), (16384, 64, 16384, False),
])
def test_quantize_bit_exact(K, N, G, sym):
    _check(_weights(K * 7 + N, K, N), G, sym, f"K={K} N={N} G={G} sym={sym}")


def test_quantize_degenerate_groups():
    K, N, G = 64, 16, 32
    W = _weights(5, K, N).copy()
    W[:, 0] = 0                                # all-zero column
    W[:, 1] = 0x3800                           # constant 0.5
    W[:, 2] = 0xB400                           # constant -0.25
    W[:G, 3] = 0x3C00                          # first group constant, second random
    W[:, 4] = 0x8000                           # negative zeros
    for sym in (False, True):
        _check(W, G, sym, f"degenerate sym={sym}")


def test_quantize_llama_layer_and_run():
    """A 4096 x 14336 layer (decode gate shape) quantized on the GPU, bit-exact,
    then multiplied by the fused GEMV against the oracle's layer of the same codes."""
    K, N, G = 4096, 14336, 128
    W = _weights(11, K, N, spread=False)
    codes, S, Z, lay = _check(W, G, False, "llama gate")
    X = synth.make_x(1, K, 99)
    o = oracle.load()
    Wq = o.dequant(o.pack(codes), S, o.pack_zeros(Z), G)
    _, Y16 = o.matmul_w(X, Wq)
    y = to_host_bits(binding.gemv(to_dev(X), lay))
    torch.cuda.synchronize()
    assert_y_close(y, Y16, "gemv on the GPU-quantized layer")


def test_quantize_exact_ties():
    """Every group spans exactly 15 s with s a power of two, and its other
    weights sit on half steps (j + 1/2) s: each w / s is an exact tie, which the
    kernel must round like the correctly rounded quotient (ties to even)."""
    K, N, G = 256, 64, 32
    rng = np.random.default_rng(31)
    W = np.zeros((K, N), dtype=np.float64)
    for g in range(K // G):
        for n in range(N):
            s = 2.0 ** -int(rng.integers(3, 12))
            z = int(rng.integers(0, 16))                       # lo = -z s, hi = (15 - z) s
            vals = (rng.integers(-z, 15 - z, G) + 0.5) * s     # half steps inside the range
            vals[0], vals[1] = -z * s, (15 - z) * s
            W[g * G:(g + 1) * G, n] = vals
    W16 = W.astype(np.float16)
    assert np.array_equal(W16.astype(np.float64), W)          # all exact in fp16
    codes, _, _, _ = _check(W16.view(np.uint16), G, False, "exact ties")
    assert codes.max() <= 15


def test_quantize_scale_rounded_once():
    """Groups whose exact range / 15 rounds differently from the same range or
    quotient formed in fp32: hi = 693.5, lo = -0.015594482421875 (exact scale
    46.21875, 0x51C7; 46.25 through fp32), and the first such pairs of a seeded
    draw of fp16 extremes.  Symmetric: every positive finite fp16 max|w|."""
    rng = np.random.default_rng(34)
    a = rng.integers(0, 0x7C00, 1 << 21).astype(np.uint16)
    b = rng.integers(0, 0x7C00, 1 << 21).astype(np.uint16) | np.uint16(0x8000)
    fa = a.view(np.float16).astype(np.float32)
    fb = b.view(np.float16).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        f32 = ((fa - fb) / np.float32(15)).astype(np.float16).view(np.uint16)
        f64 = ((fa.astype(np.float64) - fb) / 15.0).astype(np.float16).view(np.uint16)
    pick = np.nonzero((f32 != f64) & np.isfinite(fa - fb))[0][:248]
    hi = np.concatenate([[np.float16(693.5).view(np.uint16)], a[pick], a[:255 - len(pick)]])
    lo = np.concatenate([[np.float16(-0.015594482421875).view(np.uint16)], b[pick],
                         b[:255 - len(pick)]])
    N = len(hi)
    assert N % 8 == 0
    W = np.empty((16, N), dtype=np.uint16)
    W[0], W[1:8] = hi, lo                 # group 0: extremes hi, lo
    W[8:] = hi                            # group 1: constant hi
    W[9] = lo                             #          ... with one lo row
    codes, S, Z, _ = _check(W, 8, False, "scale rounded once")
    assert int(S[0][0]) == 0x51C7

    amax = np.arange(1, 0x7C00, dtype=np.uint16)
    amax = np.concatenate([amax, np.zeros((-len(amax)) % 8, dtype=np.uint16)])
    W = np.zeros((8, len(amax)), dtype=np.uint16)
    W[0] = amax
    W[1] = amax | 0x8000                  # -max|w| in the same group
    _check(W, 8, True, "symmetric scale, every max|w|")


@pytest.mark.parametrize("sym", [False, True])
def test_quantize_subnormal_scales_and_run(sym):
    """Groups whose range is below 15 * 2^-14 get subnormal fp16 scales
    (about 7e-6 here): codes, scales and zeros bit-exact, then the layer
    through awq_gemv (1 and 16 rows) and awq_gemm (64 rows) against the
    oracle's layer built from the same codes."""
    K, N, G = 2048, 1024, 128
    rng = np.random.default_rng(57)
    W = (rng.standard_normal((K, N)) * 2e-5).astype(np.float16).view(np.uint16)
    codes, S, Z, lay = _check(W, G, sym, f"subnormal scales sym={sym}")
    assert np.mean((S & 0x7C00) == 0) > 0.99                   # subnormal (or zero) scales
    o = oracle.load()
    Wq = o.dequant(o.pack(codes), S, None if sym else o.pack_zeros(Z), G)
    for fn, M in ((binding.gemv, 1), (binding.gemv, 16), (binding.gemm, 64)):
        X = synth.make_x(M, K, 58 + M)
        _, Y16 = o.matmul_w(X, Wq)
        y = to_host_bits(fn(to_dev(X), lay))
        torch.cuda.synchronize()
        assert_y_close(y, Y16, f"{fn.__name__} M={M} on subnormal scales sym={sym}")
