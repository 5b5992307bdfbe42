"""A seeded sweep of layer shapes through every layer entry point, on both word
layouts, against the oracle.

Each case draws a group size (8 to 256, or one group), K (a multiple of it),
N (a multiple of 8, of 128 for blocked words), the symmetric or asymmetric
form, the word layout (canonical, interleaved or blocked) and a batch, so that the launchers' choices -- strip widths, staging modes, uneven
segment splits, tile heights and step sizes, the general paths -- are crossed
with one another rather than exercised one shape at a time.  Shapes the
documented rules exclude are expected to be rejected with their status, not
run.  Every output is compared with the oracle under the layer's bar.
"""
import numpy as np
import pytest

from gpu_cases import device_case, oracle_case, random_case
from parity import assert_y_close, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding

import oracle

pytestmark = pytest.mark.gpu

N_CASES = 120


def draw_case(seed):
    rng = np.random.default_rng(10_000 + seed)
    G = int(rng.choice([8, 16, 32, 64, 128, 256, 0]))
    if G == 0:                                   # one group per column
        K = int(rng.choice([64, 128, 256, 512, 1024, 2048]))
        G = K
    else:
        K = G * int(rng.integers(1, max(2, 4096 // G) + 1))
        K = min(K, 4096 - 4096 % G)
    N = 8 * int(rng.integers(1, 257))            # 8 .. 2048
    sym = bool(rng.integers(0, 2))
    layout = int(rng.integers(0, 2))
    if layout and seed % 3 == 0:                 # blocked words: N a multiple of 128
        N, layout = 128 * max(1, N // 128), 2
    m_gemv = int(rng.integers(1, 17))
    m_gemm = int(rng.choice([1, 3, 16, 33, 64, 130, 257, 600]))
    return K, N, G, sym, layout, m_gemv, m_gemm


def _layer(seed, M, K, N, G, sym, layout):
    X, codes, zeros, scales = random_case(20_000 + seed, M, K, N, G, sym)
    lay = device_case(codes, zeros, scales, G)
    if layout:
        lay = binding.repack(lay, layout)
    return X, codes, zeros, scales, lay


@pytest.mark.parametrize("seed", range(N_CASES))
def test_sweep(seed):
    K, N, G, sym, layout, m_gemv, m_gemm = draw_case(seed)
    M = max(m_gemv, m_gemm)
    print(f"sweep {seed}: K={K} N={N} G={G} sym={sym} layout={layout} gemv M={m_gemv} "
          f"gemm M={m_gemm}", flush=True)
    X, codes, zeros, scales, lay = _layer(seed, M, K, N, G, sym, layout)
    _, Y16 = oracle_case(X, codes, zeros, scales, G)
    tag = f"seed {seed} K={K} N={N} G={G} sym={sym} layout={layout}"

    y = to_host_bits(binding.gemv(to_dev(X[:m_gemv]), lay))
    assert_y_close(y, Y16[:m_gemv], f"gemv M={m_gemv} {tag}")

    x = to_dev(X[:m_gemm])
    y = to_host_bits(binding.gemm(x, lay))
    assert_y_close(y, Y16[:m_gemm], f"gemm M={m_gemm} {tag}")

    splits = binding.splitk_splits(m_gemm, lay)
    if splits > 1:
        y = to_host_bits(binding.gemm_splitk(x, lay, splits))
        assert_y_close(y, Y16[:m_gemm], f"gemm_splitk M={m_gemm} splits={splits} {tag}")

    # the fused gate/up forms, where their rules take the layer ([gate | up] columns)
    if N % 16 == 0 and (G % 128 == 0 or (G % 64 == 0 and K % 256 == 0)):
        o = oracle.load()
        W, _ = oracle_case(np.zeros((1, K), np.uint16), codes, zeros, scales, G)
        H = o.gate_up(o.matmul_w(X[:M], W)[0])
        if G % 128 == 0:
            h = to_host_bits(binding.gemv_gate_up(to_dev(X[:m_gemv]), lay))
            assert_y_close(h, H[:m_gemv], f"gemv_gate_up M={m_gemv} {tag}")
        if G % 64 == 0 and K % 256 == 0:
            h = to_host_bits(binding.gemm_gate_up(x, lay))
            assert_y_close(h, H[:m_gemm], f"gemm_gate_up M={m_gemm} {tag}")


def test_sweep_covers_the_launchers():
    """The drawn cases span the group sizes, one-group layers, both forms and
    both layouts, and batches on both sides of 16 and of 64 rows."""
    cases = [draw_case(s) for s in range(N_CASES)]
    assert {c[2] for c in cases if c[2] != c[0]} >= {8, 32, 64, 128}
    assert any(c[2] == c[0] for c in cases)
    assert {c[3] for c in cases} == {False, True} and {c[4] for c in cases} == {0, 1, 2}
    assert any(c[6] <= 16 for c in cases) and any(c[6] > 64 for c in cases)
    assert max(c[0] for c in cases) >= 2048 and max(c[1] for c in cases) >= 1024
