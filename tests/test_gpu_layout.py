"""GPU parity of the kernel-private interleaved layout (AWQ_LAYOUT_INTERLEAVED).

* awq_repack against the oracle's permutation (oracle_interleave /
  oracle_deinterleave), bit for bit, both directions and in place.
* Every entry point on a repacked layer against the same entry point on the
  canonical layer: the exact ones (awq_dequant, and every GEMM path: the
  dequantized weights are the same bits and each output's sum runs over k in
  the same order) bit for bit, the GEMV within the layer's tolerance of the
  oracle (its fold reads the codes in another k order inside the matrix-core
  instruction), one-hot rows bit for bit.
Shapes cover each kernel family: 256-, 128- and 64-row GEMM tiles, 32- and
64-k steps, one group per column, symmetric zeros, the general GEMM path, split
K (workspace and static scratch), the fused gate/up forms, and the decode
kernels (staged X at 1-4 rows, X staged per segment beyond, narrow strips, the
folded and exact kernels).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_cases import device_case, oracle_case, random_case
from parity import assert_y_close, same_halves_up_to_zero_sign, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding

pytestmark = pytest.mark.gpu
IL = binding.LAYOUT_INTERLEAVED


@pytest.mark.parametrize("K,N", [(8, 8), (64, 24), (4096, 14336), (136, 200)])
def test_repack_matches_oracle(K, N):
    rng = np.random.default_rng(K + N)
    Q = rng.integers(-(1 << 31), 1 << 31, (K // 8, N), dtype=np.int64).astype(np.int32)
    o = oracle.load()
    q = to_dev(Q)
    il = binding.repack_words(q, IL)
    assert np.array_equal(il.cpu().numpy(), o.interleave(Q))
    back = binding.repack_words(il, binding.LAYOUT_CANONICAL, frm=IL)
    assert np.array_equal(back.cpu().numpy(), Q)
    binding.repack_words(q, IL, out=q)                  # in place
    assert np.array_equal(q.cpu().numpy(), o.interleave(Q))
    de = binding.repack_words(to_dev(Q), binding.LAYOUT_CANONICAL, frm=IL)
    assert np.array_equal(de.cpu().numpy(), o.deinterleave(Q))


def _pair(seed, M, K, N, G, sym):
    X, codes, zeros, scales = random_case(seed, M, K, N, G, sym)
    lay = device_case(codes, zeros, scales, G)
    return X, codes, zeros, scales, lay, binding.repack(lay, IL)


@pytest.mark.parametrize("K,N,G,sym", [(256, 136, 64, False), (512, 72, 8, True), (1024, 40, 1024, False)])
def test_dequant_interleaved_bit_exact(K, N, G, sym):
    _, codes, zeros, scales, lay, lil = _pair(7 + K, 1, K, N, G, sym)
    W, _ = oracle_case(np.zeros((1, K), np.uint16), codes, zeros, scales, G)
    assert np.array_equal(to_host_bits(binding.dequant(lil)), W)
    assert np.array_equal(to_host_bits(binding.dequant(lay)), W)


GEMM_CASES = [
    # M, K, N, G, sym: path
    (2200, 384, 14584, 128, False),   # 256-row tiles, 32-k steps
    (300, 4096, 520, 128, False),     # 128-row tiles, 64-k steps
    (50, 2048, 200, 128, True),       # 64-row tiles, symmetric
    (130, 640, 264, 32, False),       # 32-k steps
    (65, 896, 136, 64, False),
    (2200, 512, 14584, 512, False),   # one group per column (scale after the sum)
    (300, 1024, 136, 1024, True),
    (37, 200, 136, 8, False),         # general path
    (257, 1024, 8, 128, False),
]


@pytest.mark.parametrize("M,K,N,G,sym", GEMM_CASES)
def test_gemm_interleaved_bit_identical(M, K, N, G, sym):
    X, codes, zeros, scales, lay, lil = _pair(300 + M + K, M, K, N, G, sym)
    x = to_dev(X)
    a = to_host_bits(binding.gemm(x, lay))
    b = to_host_bits(binding.gemm(x, lil))
    torch.cuda.synchronize()
    assert np.array_equal(a, b), f"M={M} K={K} N={N} G={G}: {int(np.sum(a != b))} outputs differ"
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 14)])
    _, Y16 = oracle_case(X, codes, zeros, scales, G, rows=rows)
    assert_y_close(b[rows], Y16, f"interleaved gemm M={M} K={K} N={N} G={G}")


@pytest.mark.parametrize("M,K,N,G,splits", [(64, 4096, 4096, 128, 4), (200, 2048, 520, 128, 2),
                                            (48, 4096, 1032, 4096, 8)])
def test_splitk_interleaved_bit_identical(M, K, N, G, splits):
    X, _, _, _, lay, lil = _pair(400 + M, M, K, N, G, False)
    x = to_dev(X)
    a = to_host_bits(binding.gemm_splitk(x, lay, splits))
    b = to_host_bits(binding.gemm_splitk(x, lil, splits))
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    c = to_host_bits(binding.gemm_splitk_static(x, lil, splits, out))
    torch.cuda.synchronize()
    assert np.array_equal(a, b) and np.array_equal(a, c)


@pytest.mark.parametrize("M", [16, 130])
def test_gemm_gate_up_interleaved_bit_identical(M):
    X, _, _, _, lay, lil = _pair(500 + M, M, 1024, 512, 128, False)
    x = to_dev(X)
    a = to_host_bits(binding.gemm_gate_up(x, lay))
    b = to_host_bits(binding.gemm_gate_up(x, lil))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)


GEMV_CASES = [
    # M, K, N, G, sym: kernel family
    (1, 4096, 14336, 128, False),     # decode: X staged up front
    (3, 2048, 1032, 256, True),
    (4, 4096, 520, 4096, False),      # one group per column
    (7, 4096, 200, 256, True),        # X staged per segment
    (16, 4096, 1032, 128, False),
    (16, 4096, 4096, 128, False),     # narrow: 32-column strips
    (1, 4096, 4096, 128, False),
    (3, 28672, 264, 128, False),      # up to four rows, X beyond LDS
    (2, 96, 40, 32, False),           # folded kernel
    (5, 256, 72, 64, False),
    (3, 136, 200, 8, False),          # exact kernel
]


@pytest.mark.parametrize("M,K,N,G,sym", GEMV_CASES)
def test_gemv_interleaved_parity(M, K, N, G, sym):
    X, codes, zeros, scales, lay, lil = _pair(600 + M + K + N, M, K, N, G, sym)
    print(f"interleaved gemv M={M} K={K} N={N} G={G} sym={sym}", flush=True)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    y = to_host_bits(binding.gemv(to_dev(X), lil))
    torch.cuda.synchronize()
    assert_y_close(y, Y16, f"interleaved gemv M={M} K={K} N={N} G={G} sym={sym}")


@pytest.mark.parametrize("K,N,G,sym", [(4096, 1024, 128, False), (1024, 136, 1024, True),
                                       (256, 200, 8, False), (512, 512, 32, False)])
def test_gemv_interleaved_onehot_bit_exact(K, N, G, sym):
    _, codes, zeros, scales, lay, lil = _pair(5 + K, 1, K, N, G, sym)
    W, _ = oracle_case(np.zeros((1, K), np.uint16), codes, zeros, scales, G)
    ks = np.random.default_rng(K + N).choice(K, size=16, replace=False)
    for rows in (1, 4, 16):
        X = np.zeros((rows, K), dtype=np.uint16)
        X[np.arange(rows), ks[:rows]] = 0x3C00
        y = to_host_bits(binding.gemv(to_dev(X), lil))
        assert same_halves_up_to_zero_sign(y, W[ks[:rows]]), rows


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemv_gate_up_interleaved(M):
    K, N, G = 4096, 1024, 128
    X, codes, zeros, scales, lay, lil = _pair(700 + M, M, K, N, G, False)
    o = oracle.load()
    W, _ = oracle_case(np.zeros((1, K), np.uint16), codes, zeros, scales, G)
    Y64, _ = o.matmul_w(X, W)
    H = o.gate_up(Y64)
    h = to_host_bits(binding.gemv_gate_up(to_dev(X), lil))
    torch.cuda.synchronize()
    assert_y_close(h, H, f"interleaved gate/up M={M}")
