"""Every code, zero point and finite fp16 scale through the fused kernels.

awq_dequant is already checked bit for bit on every (q, z, s); here the same
exhaustive layers go through the multiplying kernels, with inputs for which
each output receives exactly one nonzero product (x = 1), so the output must
be the dequantized weight fp16_rne(s (q - z)) bit for bit, up to the sign of
zero (fak explainer, "Format Specification > Dequantization Formula"; the
reading w = fp16(s (q - z)) rounded once):

* awq_gemm with X = I_K, on the exact-dequantization paths (G = 32 and 64:
  32-k and 64-k steps) and on the one-group path (G = K, where the scale
  multiplies the fp32 sum of q - z);
* awq_gemv with one-hot rows, at 1 row (the decode kernel) and 16 rows, on a
  G = 128 layer (the staged kernels) and a G = 32 layer (the folded kernel).

Scales cover all 63,488 finite fp16 patterns: negative ones, zeros,
subnormals, and the largest, where s (q - z) overflows to infinity.  In the
exact-dequantization GEMM a column that holds an infinite weight has
0 * inf = NaN in every other row (the oracle's plain sum has the same NaN),
so there only the columns whose weights are all finite are compared; every
other kernel here never forms a weight before the multiply and is compared
everywhere, infinities included.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import same_halves_up_to_zero_sign, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding

pytestmark = pytest.mark.gpu

ALL_H = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE = ALL_H[(ALL_H & 0x7C00) != 0x7C00]          # 63,488 patterns, N % 8 == 0


def _grouped_layer(G, groups, sym):
    """Row k has code k % 16, group g has zero g, column n scale FINITE[n]."""
    K = G * groups
    N = FINITE.size
    codes = np.tile((np.arange(K) % 16).astype(np.uint8)[:, None], (1, N))
    zeros = None if sym else np.tile(np.arange(groups, dtype=np.uint8)[:, None] % 16, (1, N))
    scales = np.ascontiguousarray(np.tile(FINITE[None, :], (groups, 1)))
    return codes, zeros, scales


def _one_group_layer(K, sym):
    """One group per column (G = K): column n has scale FINITE[n // 16] and
    zero n % 16 (asymmetric), or scale FINITE[n] (symmetric)."""
    reps = 1 if sym else 16
    N = FINITE.size * reps
    codes = np.tile((np.arange(K) % 16).astype(np.uint8)[:, None], (1, N))
    scales = np.repeat(FINITE, reps)[None, :].copy()
    zeros = None if sym else (np.arange(N) % 16).astype(np.uint8)[None, :].copy()
    return codes, zeros, scales


def _weights(codes, zeros, scales, G):
    o = oracle.load()
    return o.dequant(o.pack(codes), scales, None if zeros is None else o.pack_zeros(zeros), G)


def _device(codes, zeros, scales, G):
    return binding.make_layer(to_dev(codes), None if zeros is None else to_dev(zeros),
                              to_dev(scales), G)


def _finite_columns(W):
    return np.all((W & 0x7C00) != 0x7C00, axis=0)


@pytest.mark.parametrize("G,groups,sym", [(32, 16, False), (64, 16, False), (32, 4, True),
                                          (64, 4, True)])
def test_gemm_identity_every_scale(G, groups, sym):
    codes, zeros, scales = _grouped_layer(G, groups, sym)
    K = codes.shape[0]
    print(f"gemm identity: K={K} N={codes.shape[1]} G={G} sym={sym}", flush=True)
    W = _weights(codes, zeros, scales, G)
    X = np.zeros((K, K), dtype=np.uint16)
    X[np.arange(K), np.arange(K)] = 0x3C00
    y = to_host_bits(binding.gemm(to_dev(X), _device(codes, zeros, scales, G)))
    torch.cuda.synchronize()
    fin = _finite_columns(W)
    assert fin.sum() >= 0.85 * fin.size           # only the largest scales overflow
    assert same_halves_up_to_zero_sign(y[:, fin], W[:, fin])


@pytest.mark.parametrize("sym", [False, True])
def test_gemm_identity_every_scale_one_group(sym):
    K = 128
    codes, zeros, scales = _one_group_layer(K, sym)
    print(f"gemm identity, one group: K={K} N={codes.shape[1]} sym={sym}", flush=True)
    W = _weights(codes, zeros, scales, K)
    X = np.zeros((K, K), dtype=np.uint16)
    X[np.arange(K), np.arange(K)] = 0x3C00
    y = to_host_bits(binding.gemm(to_dev(X), _device(codes, zeros, scales, K)))
    torch.cuda.synchronize()
    assert np.any((W & 0x7FFF) == 0x7C00)          # overflowing products are covered
    assert same_halves_up_to_zero_sign(y, W)


@pytest.mark.parametrize("G,rows", [(128, 1), (128, 16), (32, 16)])
def test_gemv_onehot_every_scale(G, rows):
    """Rows k = g G + q (q = 0..15) of every group g: each (q, z, s) once."""
    groups = 16
    codes, zeros, scales = _grouped_layer(G, groups, False)
    K = codes.shape[0]
    print(f"gemv one-hot: K={K} N={codes.shape[1]} G={G} rows per call={rows}", flush=True)
    W = _weights(codes, zeros, scales, G)
    layer = _device(codes, zeros, scales, G)
    ks = (np.arange(groups)[:, None] * G + np.arange(16)[None, :]).ravel()
    for c in range(0, ks.size, rows):
        sel = ks[c:c + rows]
        X = np.zeros((sel.size, K), dtype=np.uint16)
        X[np.arange(sel.size), sel] = 0x3C00
        y = to_host_bits(binding.gemv(to_dev(X), layer))
        assert same_halves_up_to_zero_sign(y, W[sel]), f"rows {sel[0]}..{sel[-1]}"
