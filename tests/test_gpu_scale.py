"""GPU parity of the scale search (awq_channel_stats, awq_scale_search) against
the oracle.

The statistics are fp64 sums on both sides (the GPU divides |w| by the group
maximum in fp32), so they agree to fp32 rounding.  The candidate scales use the
GPU's fp32 powf against the oracle's fp64 pow, so a migrated weight can round
to the other fp16 neighbour in rare places, and the candidate's output is the
fused GEMM's fp32 sum against the oracle's fp64 sum; each loss is therefore
held to 1% of the oracle's, and the GPU's choice must be a least loss of the
oracle's within that margin (where several alphas are that close, any of them
is correct).  The inputs follow the calibration recipe: X ~ N(0, 1) with 1% of
its channels scaled by 20 (the outlier channels the method protects), W ~ N(0,
0.02), some weight groups all zero.
"""
import numpy as np
import pytest
import torch

from parity import to_dev
from w4a16_group_quantized_amd import binding

import oracle

pytestmark = pytest.mark.gpu

ALPHAS = [0.0, 0.25, 0.5, 0.75, 1.0]


def _calibration(seed, M, K, N, G):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    hot = rng.choice(K, size=max(1, K // 100), replace=False)
    X[:, hot] *= 20.0
    W = rng.standard_normal((K, N)) * 0.02
    if K // G > 1:
        W[:G, : N // 4] = 0.0                       # all-zero groups: they add 0 to wbar
    return X.astype(np.float16).view(np.uint16), W.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("M,K,N,G", [(96, 256, 136, 64), (300, 512, 64, 512), (1, 128, 8, 8),
                                     (130, 1024, 200, 128)])
def test_channel_stats(M, K, N, G):
    X, W = _calibration(M + K, M, K, N, G)
    xbar, wbar = binding.channel_stats(to_dev(X), to_dev(W), G)
    torch.cuda.synchronize()
    ox, ow = oracle.load().channel_stats(X, W, G)
    for got, want, what in ((xbar, ox, "xbar"), (wbar, ow, "wbar")):
        got = got.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - want) <= 1e-6 * np.abs(want) + 1e-30), what


@pytest.mark.parametrize("M,K,N,G,sym", [
    (64, 256, 128, 64, False), (48, 512, 72, 128, True), (32, 384, 64, 384, False),
    (128, 4096, 512, 128, False),
    # long groups: the migrating quantizer with 8 waves a group
    (64, 2048, 136, 1024, False), (32, 4096, 72, 4096, True),
])
def test_scale_search(M, K, N, G, sym):
    X, W = _calibration(7 * M + K, M, K, N, G)
    alphas = ALPHAS if K < 4096 else [0.0, 0.5, 1.0]
    best, losses, scales = binding.scale_search(to_dev(X), to_dev(W), G, alphas, sym)
    torch.cuda.synchronize()
    o = oracle.load()
    obest, olosses, oc = o.scale_search(X, W, G, sym, alphas)
    losses = losses.cpu().numpy()
    rel = np.abs(losses - olosses) / olosses
    assert np.all(rel <= 1e-2), (losses, olosses)
    b = int(best.item())
    assert olosses[b] <= olosses.min() * (1 + 1e-2), (b, obest, olosses)
    xbar, wbar = o.channel_stats(X, W, G)
    want = o.scale_candidate(xbar, wbar, alphas[b])
    got = scales.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-5 * want), "scales of the chosen alpha"


def test_scale_search_deterministic():
    X, W = _calibration(3, 64, 512, 96, 128)
    x, w = to_dev(X), to_dev(W)
    runs = [binding.scale_search(x, w, 128, ALPHAS)[1].cpu().numpy() for _ in range(3)]
    assert all(np.array_equal(runs[0], r) for r in runs[1:])


def test_scale_search_all_equal_keeps_first():
    """|x| = 1 and |w| constant within each group and column: every alpha gives
    c = 1, every loss is the same, and the first alpha is kept."""
    rng = np.random.default_rng(5)
    M, K, N, G = 32, 256, 64, 64
    X = rng.choice([-1.0, 1.0], (M, K)).astype(np.float16).view(np.uint16)
    a = np.repeat(np.ldexp(1.0, rng.integers(-8, -2, (K // G, N))), G, axis=0)
    W = (a * rng.choice([-1.0, 1.0], (K, N))).astype(np.float16).view(np.uint16)
    best, losses, scales = binding.scale_search(to_dev(X), to_dev(W), G, ALPHAS)
    torch.cuda.synchronize()
    losses = losses.cpu().numpy()
    assert int(best.item()) == 0
    assert np.all(losses == losses[0])
    assert np.all(scales.cpu().numpy() == 1.0)
    _, olosses, _ = oracle.load().scale_search(X, W, G, False, ALPHAS)
    assert abs(losses[0] - olosses[0]) <= 1e-2 * olosses[0]


def test_scale_search_given_workspace_reused():
    """A caller-owned workspace serves two searches in a row (the second one
    smaller); its contents between calls do not matter."""
    lib = binding.load()
    nbytes = lib.awq_scale_search_workspace_bytes(64, 512, 96, 128)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for (M, K, N, G) in ((64, 512, 96, 128), (16, 256, 32, 64)):
        X, W = _calibration(M, M, K, N, G)
        _, losses, _ = binding.scale_search(to_dev(X), to_dev(W), G, ALPHAS, workspace=ws)
        torch.cuda.synchronize()
        _, olosses, _ = oracle.load().scale_search(X, W, G, False, ALPHAS)
        assert np.all(np.abs(losses.cpu().numpy() - olosses) <= 1e-2 * olosses)
