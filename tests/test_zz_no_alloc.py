"""awq_gemm_splitk_static, the split-K GEMM on the library's static scratch
(no allocation in the call), against awq_gemm_splitk with a caller workspace:
the same kernels, so the outputs must match bit for bit.  Two calls in a row,
the second with a smaller input (the scratch keeps the first call's partial
sums, which the second must not read), then an oversized request, which is
rejected before any launch.  Also checked against the oracle to the layer's
tolerance.
"""
import numpy as np
import pytest
import torch

from gpu_cases import device_case, oracle_case, random_case
from parity import assert_y_close, to_dev, to_host_bits
from w4a16_group_quantized_amd import binding

pytestmark = pytest.mark.gpu


def _run(seed, M, K, N, G, splits, sym=False):
    X, codes, zeros, scales = random_case(seed, M, K, N, G, sym)
    lay = device_case(codes, zeros, scales, G)
    x = to_dev(X)
    print(f"no-alloc split-K: seed={seed} M={M} K={K} N={N} G={G} splits={splits}", flush=True)
    out_static = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    binding.gemm_splitk_static(x, lay, splits, out_static)
    ref = binding.gemm_splitk(x, lay, splits=splits)
    torch.cuda.synchronize()
    a, b = to_host_bits(out_static), to_host_bits(ref)
    assert np.array_equal(a, b), f"M={M} splits={splits}: static scratch differs from the workspace call"
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(seed).integers(0, M, 6)])
    _, Y16 = oracle_case(X, codes, zeros, scales, G, rows=rows)
    assert_y_close(a[rows], Y16, f"static split-K M={M}")


def test_static_scratch_two_calls_then_smaller():
    _run(71, 256, 4096, 4096, 128, 4)          # 16 MiB of partials
    _run(72, 16, 4096, 4096, 128, 8)           # smaller: 2 MiB, over the first call's leftovers
    _run(73, 37, 2048, 136, 2048, 2, sym=True)  # ragged rows and columns, one group


def test_static_scratch_too_small_is_rejected():
    K, N, G = 4096, 28672, 128
    X, codes, zeros, scales = random_case(74, 128, K, N, G, False)
    lay = device_case(codes, zeros, scales, G)
    out = torch.empty((128, N), dtype=torch.float16, device="cuda")
    assert 4 * 128 * N * 4 > binding.GEMM_SPLITK_STATIC_SCRATCH_BYTES
    with pytest.raises(binding.AwqError) as e:
        binding.gemm_splitk_static(to_dev(X), lay, 4, out)
    assert e.value.status == binding.AWQ_ERROR_WORKSPACE
