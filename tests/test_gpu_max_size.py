"""The largest layer the C ABI takes: K * N just below 2^31 elements.

K = 8192 and N = 262136 give K N = 2,147,418,112 (a 1.07 GB packed weight, a
4.3 GB dequantized one), so every index and byte offset the kernels form on
this layer sits near the top of its range: 32-bit buffer sizes, per-step
offsets, and the dequantized output's 64-bit addressing.  The packed words, the
scales and the zero points are seeded host draws (uniform words, scales in
[0.001, 0.01]); the oracle takes the same host arrays, restricted to seeded
blocks of 8 columns across the whole width (always the first and the last),
and computes those columns.  Rows of X come from the synthetic generator.
Each kernel variant the shapes select is covered: the decode kernel at 1 row
and in its slot-staged form at 16 rows (X staged segment by segment), the GEMM,
split K and the exact dequantization.  The same again on blocked words, whose
N must be a multiple of 128: N = 262016, the largest such width under 2^31 /
K, repacked on the GPU from the seeded canonical words.  Two more cases take
the largest batch (M K just below 2^31, a 4.3 GB X through the GEMM) and the
largest fp16 W through the quantizer.
"""
import numpy as np
import pytest
import torch

from parity import assert_y_close, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding, synth

import oracle

pytestmark = pytest.mark.gpu

K, N, G = 8192, 262136, 128


@pytest.fixture(scope="module")
def big():
    rng = np.random.default_rng(20261203)
    Q = rng.integers(0, 1 << 32, size=(K // 8, N), dtype=np.uint32).view(np.int32)
    S = rng.uniform(0.001, 0.01, size=(K // G, N)).astype(np.float16).view(np.uint16)
    QZ = rng.integers(0, 1 << 32, size=(K // G, N // 8), dtype=np.uint32).view(np.int32)
    layer = binding.Layer(torch.from_numpy(Q).cuda(), torch.from_numpy(S.view(np.float16)).cuda(),
                          torch.from_numpy(QZ).cuda(), K, N, G)
    blocks = np.array(sorted({0, N // 8 - 1} | set(rng.choice(N // 8, 30, replace=False).tolist())))
    cols = (8 * blocks[:, None] + np.arange(8)[None, :]).reshape(-1)
    sampled = (np.ascontiguousarray(Q[:, cols]), np.ascontiguousarray(S[:, cols]),
               np.ascontiguousarray(QZ[:, blocks]))
    yield layer, cols, sampled
    del layer
    torch.cuda.empty_cache()


NB = 262016   # the largest multiple of 128 with K * NB below 2^31


@pytest.fixture(scope="module")
def big_blocked():
    rng = np.random.default_rng(20261204)
    Q = rng.integers(0, 1 << 32, size=(K // 8, NB), dtype=np.uint32).view(np.int32)
    S = rng.uniform(0.001, 0.01, size=(K // G, NB)).astype(np.float16).view(np.uint16)
    QZ = rng.integers(0, 1 << 32, size=(K // G, NB // 8), dtype=np.uint32).view(np.int32)
    canon = binding.Layer(torch.from_numpy(Q).cuda(), torch.from_numpy(S.view(np.float16)).cuda(),
                          torch.from_numpy(QZ).cuda(), K, NB, G)
    layer = binding.repack(canon, binding.LAYOUT_BLOCKED)
    del canon
    torch.cuda.empty_cache()
    blocks = np.array(sorted({0, 15, 16, NB // 8 - 1} |
                             set(rng.choice(NB // 8, 30, replace=False).tolist())))
    cols = (8 * blocks[:, None] + np.arange(8)[None, :]).reshape(-1)
    sampled = (np.ascontiguousarray(Q[:, cols]), np.ascontiguousarray(S[:, cols]),
               np.ascontiguousarray(QZ[:, blocks]))
    yield layer, cols, sampled
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("entry,M", [("gemv", 1), ("gemv", 16), ("gemm", 64), ("splitk", 64),
                                     ("dequant", 0)])
def test_largest_blocked_layer(big_blocked, entry, M):
    layer, cols, sampled = big_blocked
    print(f"largest blocked layer: {entry} M={M}", flush=True)
    ci = torch.from_numpy(cols).cuda()
    if entry == "dequant":
        W = binding.dequant(layer)
        torch.cuda.synchronize()
        got = to_host_bits(W[:, ci])
        del W
        torch.cuda.empty_cache()
        Qs, Ss, QZs = sampled
        assert np.array_equal(got, oracle.load().dequant(Qs, Ss, QZs, G))
        return
    X = synth.make_x(M, K, 700 + M)
    if entry == "splitk":
        y = binding.gemm_splitk(to_dev(X), layer, 4)
    else:
        y = (binding.gemv if entry == "gemv" else binding.gemm)(to_dev(X), layer)
    torch.cuda.synchronize()
    got = to_host_bits(y[:, ci])
    assert_y_close(got, _oracle_y(X, sampled), f"{entry} M={M} on the largest blocked layer")


def _oracle_y(X, sampled):
    Qs, Ss, QZs = sampled
    return oracle.load().linear(X, Qs, Ss, QZs, G)[1]


@pytest.mark.parametrize("entry,M", [("gemv", 1), ("gemv", 16), ("gemm", 64)])
def test_largest_layer(big, entry, M):
    layer, cols, sampled = big
    X = synth.make_x(M, K, 500 + M)
    fn = binding.gemv if entry == "gemv" else binding.gemm
    y = fn(to_dev(X), layer)
    torch.cuda.synchronize()
    got = to_host_bits(y[:, torch.from_numpy(cols).cuda()])
    assert_y_close(got, _oracle_y(X, sampled), f"{entry} M={M} on the largest layer")


def test_largest_layer_splitk(big):
    layer, cols, sampled = big
    X = synth.make_x(64, K, 601)
    y = binding.gemm_splitk(to_dev(X), layer, 4)
    torch.cuda.synchronize()
    got = to_host_bits(y[:, torch.from_numpy(cols).cuda()])
    assert_y_close(got, _oracle_y(X, sampled), "split K on the largest layer")


def test_largest_layer_dequant(big):
    layer, cols, sampled = big
    W = binding.dequant(layer)                                     # 4.3 GB of fp16
    torch.cuda.synchronize()
    got = to_host_bits(W[:, torch.from_numpy(cols).cuda()])
    del W
    torch.cuda.empty_cache()
    Qs, Ss, QZs = sampled
    assert np.array_equal(got, oracle.load().dequant(Qs, Ss, QZs, G))


def test_largest_batch_gemm():
    """M K just below 2^31 (M = 524287 rows at K = 4096: a 4.3 GB X): the GEMM's
    X addressing at the top of its 32-bit byte range.  X is a seeded block of 997
    rows tiled down the batch (997 is prime, so a wrong row offset lands on a
    different row unless it is a multiple of 997); the oracle computes the first,
    the last and seeded rows."""
    Kb, Nb, Gb = 4096, 64, 128
    M = (2**31 - 1) // Kb
    _, codes, zeros, scales = synth.workload_inputs(synth.WORKLOADS["decode_8b_gate"])
    codes, zeros, scales = codes[:, :Nb].copy(), zeros[:, :Nb].copy(), scales[:, :Nb].copy()
    block = synth.make_x(997, Kb, 4242)
    X = np.tile(block, (M // 997 + 1, 1))[:M]
    layer = binding.make_layer(to_dev(codes), to_dev(zeros), to_dev(scales), Gb)
    x = to_dev(X)
    del X
    y = binding.gemm(x, layer)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, M - 2, M - 1} |
                           set(np.random.default_rng(7).choice(M, 60, replace=False).tolist())))
    got = to_host_bits(y[torch.from_numpy(rows).cuda()])
    del x, y
    torch.cuda.empty_cache()
    o = oracle.load()
    Xr = np.ascontiguousarray(block[rows % 997])
    want = o.linear(Xr, o.pack(codes), scales, o.pack_zeros(zeros), Gb)[1]
    assert_y_close(got, want, "gemm on the largest batch")


@pytest.mark.parametrize("sym", [False, True])
def test_largest_layer_quantize(sym):
    """awq_quantize on a 4.3 GB fp16 W (K N just below 2^31): a seeded block of
    1009 columns (prime, as above) tiled across the width, W ~ N(0, 0.02); the
    codes, scales and zero points of sampled column blocks are the oracle's bit
    for bit."""
    rng = np.random.default_rng(1009 + sym)
    block = (rng.standard_normal((K, 1009)) * 0.02).astype(np.float16)
    blocks = np.array(sorted({0, N // 8 - 1} | set(rng.choice(N // 8, 30, replace=False).tolist())))
    cols = (8 * blocks[:, None] + np.arange(8)[None, :]).reshape(-1)
    w = torch.from_numpy(np.tile(block, (1, N // 1009 + 1))[:, :N].copy()).cuda()
    layer = binding.quantize(w, G, sym)
    torch.cuda.synchronize()
    del w
    ci = torch.from_numpy(cols).cuda()
    q = layer.qweight[:, ci].cpu().numpy()
    s = to_host_bits(layer.scales[:, ci])
    z = None if sym else layer.qzeros[:, torch.from_numpy(blocks).cuda()].cpu().numpy()
    del layer
    torch.cuda.empty_cache()
    o = oracle.load()
    codes, S, Z = o.quantize(np.ascontiguousarray(block[:, cols % 1009]).view(np.uint16), G, sym)
    assert np.array_equal(q, o.pack(codes))
    assert np.array_equal(s, S)
    if not sym:
        assert np.array_equal(z, o.pack_zeros(Z))
