"""GPU parity of the kernel-private blocked layout (AWQ_LAYOUT_BLOCKED: the
interleaved words with each 128-column block stored as one run).

* awq_repack against the oracle's permutations (oracle_block of the
  interleaved words), bit for bit, from and to both other layouts, and the
  in-place request across the blocked layout rejected.
* Every entry point on a blocked layer against the same entry point on the
  canonical layer: the exact ones (awq_dequant, every GEMM path) bit for bit,
  the GEMV within the layer's tolerance of the oracle, one-hot rows bit for bit.
Shapes (N a multiple of 128) cover each kernel family: 256-, 128- and 64-row
GEMM tiles with a half-used last column tile, 32- and 64-k steps, one group per
column, symmetric zeros, the general GEMM path, split K (workspace and static
scratch), the fused gate/up forms, and the decode kernels (staged X at 1-4
rows, X staged per segment beyond, narrow strips, the folded and exact
kernels).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import device_case, oracle_case, random_case
from parity import assert_y_close, same_halves_up_to_zero_sign, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding

pytestmark = pytest.mark.gpu
CANON, IL, BLK = binding.LAYOUT_CANONICAL, binding.LAYOUT_INTERLEAVED, binding.LAYOUT_BLOCKED


@pytest.mark.parametrize("K,N", [(8, 128), (64, 384), (4096, 14336), (136, 1280)])
def test_repack_blocked_matches_oracle(K, N):
    print(f"blocked repack K={K} N={N}", flush=True)
    rng = np.random.default_rng(K + 3 * N)
    Q = rng.integers(-(1 << 31), 1 << 31, (K // 8, N), dtype=np.int64).astype(np.int32)
    o = oracle.load()
    want = o.block(o.interleave(Q))
    b = binding.repack_words(to_dev(Q), BLK)
    assert np.array_equal(b.cpu().numpy().reshape(-1), want)
    b1 = binding.repack_words(to_dev(o.interleave(Q)), BLK, frm=IL)
    assert np.array_equal(b1.cpu().numpy().reshape(-1), want)
    back = binding.repack_words(b, CANON, frm=BLK)
    assert np.array_equal(back.cpu().numpy(), Q)
    back_il = binding.repack_words(b, IL, frm=BLK)
    assert np.array_equal(back_il.cpu().numpy(), o.interleave(Q))
    # a blocked array read as the canonical words of another layer: its own round trip
    again = binding.repack_words(binding.repack_words(to_dev(Q), CANON, frm=BLK), BLK)
    assert np.array_equal(again.cpu().numpy(), Q)
    q = to_dev(Q)
    with pytest.raises(binding.AwqError):
        binding.repack_words(q, BLK, out=q)                  # words move: not in place
    assert np.array_equal(q.cpu().numpy(), Q)


def _pair(seed, M, K, N, G, sym):
    X, codes, zeros, scales = random_case(seed, M, K, N, G, sym)
    lay = device_case(codes, zeros, scales, G)
    return X, codes, zeros, scales, lay, binding.repack(lay, BLK)


@pytest.mark.parametrize("K,N,G,sym", [(256, 128, 64, False), (512, 384, 8, True), (1024, 256, 1024, False)])
def test_dequant_blocked_bit_exact(K, N, G, sym):
    _, codes, zeros, scales, lay, lb = _pair(17 + K, 1, K, N, G, sym)
    W, _ = oracle_case(np.zeros((1, K), np.uint16), codes, zeros, scales, G)
    assert np.array_equal(to_host_bits(binding.dequant(lb)), W)


GEMM_CASES = [
    # M, K, N, G, sym: path
    (2200, 384, 14464, 128, False),   # 256-row tiles, 32-k steps, last column tile half used
    (300, 4096, 640, 128, False),     # 128-row tiles, 64-k steps
    (50, 2048, 256, 128, True),       # 64-row tiles, symmetric
    (130, 640, 384, 32, False),       # 32-k steps
    (65, 896, 128, 64, False),
    (2200, 512, 14464, 512, False),   # one group per column (scale after the sum)
    (300, 1024, 128, 1024, True),
    (37, 200, 384, 8, False),         # general path
]


@pytest.mark.parametrize("M,K,N,G,sym", GEMM_CASES)
def test_gemm_blocked_bit_identical(M, K, N, G, sym):
    print(f"blocked gemm M={M} K={K} N={N} G={G} sym={sym}", flush=True)
    X, codes, zeros, scales, lay, lb = _pair(310 + M + K, M, K, N, G, sym)
    x = to_dev(X)
    a = to_host_bits(binding.gemm(x, lay))
    b = to_host_bits(binding.gemm(x, lb))
    torch.cuda.synchronize()
    assert np.array_equal(a, b), f"M={M} K={K} N={N} G={G}: {int(np.sum(a != b))} outputs differ"
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 14)])
    _, Y16 = oracle_case(X, codes, zeros, scales, G, rows=rows)
    assert_y_close(b[rows], Y16, f"blocked gemm M={M} K={K} N={N} G={G}")


@pytest.mark.parametrize("M,K,N,G,splits", [(64, 4096, 4096, 128, 4), (200, 2048, 640, 128, 2),
                                            (48, 4096, 1024, 4096, 8)])
def test_splitk_blocked_bit_identical(M, K, N, G, splits):
    print(f"blocked split-K M={M} K={K} N={N} G={G} splits={splits}", flush=True)
    X, _, _, _, lay, lb = _pair(410 + M, M, K, N, G, False)
    x = to_dev(X)
    a = to_host_bits(binding.gemm_splitk(x, lay, splits))
    b = to_host_bits(binding.gemm_splitk(x, lb, splits))
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    c = to_host_bits(binding.gemm_splitk_static(x, lb, splits, out))
    torch.cuda.synchronize()
    assert np.array_equal(a, b) and np.array_equal(a, c)


@pytest.mark.parametrize("M", [16, 130])
def test_gemm_gate_up_blocked_bit_identical(M):
    X, _, _, _, lay, lb = _pair(510 + M, M, 1024, 768, 128, False)
    x = to_dev(X)
    a = to_host_bits(binding.gemm_gate_up(x, lay))
    b = to_host_bits(binding.gemm_gate_up(x, lb))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)


GEMV_CASES = [
    # M, K, N, G, sym: kernel family
    (1, 4096, 14336, 128, False),     # decode: X staged up front
    (3, 2048, 1024, 256, True),
    (4, 4096, 512, 4096, False),      # one group per column
    (7, 4096, 256, 256, True),        # X staged per segment
    (16, 4096, 1152, 128, False),
    (16, 4096, 28672, 128, False),    # 128-column strips
    (16, 4096, 4096, 128, False),     # narrow: 32-column strips
    (1, 4096, 4096, 128, False),
    (3, 28672, 256, 128, False),      # up to four rows, X beyond LDS
    (2, 96, 128, 32, False),          # folded kernel
    (5, 256, 384, 64, False),
    (3, 136, 128, 8, False),          # exact kernel
]


@pytest.mark.parametrize("M,K,N,G,sym", GEMV_CASES)
def test_gemv_blocked_parity(M, K, N, G, sym):
    print(f"blocked gemv M={M} K={K} N={N} G={G} sym={sym}", flush=True)
    X, codes, zeros, scales, lay, lb = _pair(610 + M + K + N, M, K, N, G, sym)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    y = to_host_bits(binding.gemv(to_dev(X), lb))
    torch.cuda.synchronize()
    assert_y_close(y, Y16, f"blocked gemv M={M} K={K} N={N} G={G} sym={sym}")
    # the interleaved words of the same layer give the same bits (the kernels
    # differ only in where they read each word)
    yi = to_host_bits(binding.gemv(to_dev(X), binding.repack(lay, IL)))
    torch.cuda.synchronize()
    assert np.array_equal(y, yi)


@pytest.mark.parametrize("K,N,G,sym", [(4096, 1024, 128, False), (1024, 256, 1024, True),
                                       (256, 384, 8, False), (512, 512, 32, False)])
def test_gemv_blocked_onehot_bit_exact(K, N, G, sym):
    _, codes, zeros, scales, lay, lb = _pair(15 + K, 1, K, N, G, sym)
    W, _ = oracle_case(np.zeros((1, K), np.uint16), codes, zeros, scales, G)
    ks = np.random.default_rng(K + N).choice(K, size=16, replace=False)
    for rows in (1, 4, 16):
        X = np.zeros((rows, K), dtype=np.uint16)
        X[np.arange(rows), ks[:rows]] = 0x3C00
        y = to_host_bits(binding.gemv(to_dev(X), lb))
        assert same_halves_up_to_zero_sign(y, W[ks[:rows]]), rows


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemv_gate_up_blocked(M):
    K, N, G = 4096, 1280, 128
    X, codes, zeros, scales, lay, lb = _pair(710 + M, M, K, N, G, False)
    o = oracle.load()
    W, _ = oracle_case(np.zeros((1, K), np.uint16), codes, zeros, scales, G)
    Y64, _ = o.matmul_w(X, W)
    H = o.gate_up(Y64)
    h = to_host_bits(binding.gemv_gate_up(to_dev(X), lb))
    torch.cuda.synchronize()
    assert_y_close(h, H, f"blocked gate/up M={M}")
