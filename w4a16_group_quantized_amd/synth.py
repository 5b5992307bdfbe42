"""Seeded synthetic inputs for the W4A16 group-quantized linear layer.

This module draws random numbers and nothing else: it holds none of the
layer's arithmetic (no packing, no dequantization, no product).  Both the HIP
path and the CPU oracle receive the very same arrays from it.

Random source: SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014).  Output i (0-based) of a stream
with seed ``s`` is ``mix(s + (i + 1) * 0x9E3779B97F4A7C15)`` in 64-bit
wrap-around arithmetic, which lets a stream be drawn in vectorised chunks.

Draws:
  * 4-bit integer: the top four bits, ``u >> 60``.
  * uniform real in [0, 1): ``(u >> 11) * 2**-53``.
  * standard normal: Box-Muller from two consecutive uniforms,
    ``sqrt(-2 ln(1 - U0)) * cos(2 pi U1)``.
  * fp16 values: drawn in double, then rounded to nearest-even fp16 by numpy.

Each tensor of a workload has its own stream, seeded
``((0x5EED0000 + workload_id) << 8) | tensor_id`` with tensor ids
X = 1, codes = 2, scales = 3, zeros = 4, outlier channel pick = 5.
Tensors are drawn row-major in their logical layout: X[M][K], codes[K][N],
scales[K/G][N], zeros[K/G][N].  Codes and zeros are returned unpacked (one
uint8 per 4-bit value); packing them is the library's (and the oracle's) job.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

TENSOR_X, TENSOR_CODES, TENSOR_SCALES, TENSOR_ZEROS, TENSOR_OUTLIERS = 1, 2, 3, 4, 5


def stream_seed(workload_id: int, tensor_id: int) -> int:
    return (((0x5EED0000 + int(workload_id)) << 8) | int(tensor_id)) & ((1 << 64) - 1)


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 stream ``seed``."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed) + i * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        return z ^ (z >> np.uint64(31))


class Stream:
    """Sequential reader over one SplitMix64 stream."""

    def __init__(self, seed: int):
        self.seed = int(seed)
        self.pos = 0

    def raw(self, count: int) -> np.ndarray:
        out = splitmix64(self.seed, self.pos, count)
        self.pos += count
        return out

    def nibbles(self, count: int) -> np.ndarray:
        out = np.empty(count, dtype=np.uint8)
        for a in range(0, count, _CHUNK):
            b = min(count, a + _CHUNK)
            out[a:b] = (self.raw(b - a) >> np.uint64(60)).astype(np.uint8)
        return out

    def uniform(self, count: int) -> np.ndarray:
        return (self.raw(count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)

    def normal_f16(self, count: int) -> np.ndarray:
        out = np.empty(count, dtype=np.float16)
        for a in range(0, count, _CHUNK):
            b = min(count, a + _CHUNK)
            u = self.uniform(2 * (b - a)).reshape(-1, 2)
            z = np.sqrt(-2.0 * np.log(1.0 - u[:, 0])) * np.cos(2.0 * np.pi * u[:, 1])
            out[a:b] = z.astype(np.float16)
        return out

    def uniform_f16(self, count: int, lo: float, hi: float) -> np.ndarray:
        out = np.empty(count, dtype=np.float16)
        for a in range(0, count, _CHUNK):
            b = min(count, a + _CHUNK)
            out[a:b] = (lo + (hi - lo) * self.uniform(b - a)).astype(np.float16)
        return out


def f16_bits(a: np.ndarray) -> np.ndarray:
    """View an fp16 array as its uint16 bit patterns."""
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


@dataclass(frozen=True)
class Workload:
    """One synthetic layer shape with its value distributions."""

    name: str
    wid: int            # workload id, part of every stream seed
    M: int
    K: int
    N: int
    G: int              # group size along K (G == K: one scale per column)
    symmetric: bool     # no zero tensor: zero point 8
    scale_lo: float
    scale_hi: float
    outlier_frac: float = 0.0   # share of K-channels of X scaled up
    outlier_gain: float = 1.0
    entry: str = "gemv"         # "gemv" or "gemm"

    @property
    def groups(self) -> int:
        return self.K // self.G

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.K))


# Llama-shaped layers.  The weight of the 70B-shaped layer is shared between the
# M=1 and M=4096 workloads (same workload id, same streams).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 512, 512, 128, False, 0.002, 0.02),
    "decode_8b_gate": Workload("decode_8b_gate", 2, 1, 4096, 14336, 128, False, 0.002, 0.02),
    "gate_up_m16": Workload("gate_up_m16", 3, 16, 4096, 28672, 128, False, 0.002, 0.02,
                            outlier_frac=0.01, outlier_gain=20.0),
    "prefill_out_proj": Workload("prefill_out_proj", 4, 2048, 4096, 4096, 128, False,
                                 0.001, 0.01, entry="gemm"),
    "sym70b_m1": Workload("sym70b_m1", 5, 1, 8192, 28672, 8192, True, 0.001, 0.01),
    "sym70b_m4096": Workload("sym70b_m4096", 5, 4096, 8192, 28672, 8192, True, 0.001, 0.01,
                             entry="gemm"),
}


def make_layer(K: int, N: int, G: int, symmetric: bool, scale_lo: float, scale_hi: float,
               wid: int):
    """Unpacked codes uint8[K][N], zeros uint8[K/G][N] (None if symmetric) and
    fp16 scales (uint16 bit patterns) [K/G][N]."""
    groups = K // G
    codes = Stream(stream_seed(wid, TENSOR_CODES)).nibbles(K * N).reshape(K, N)
    scales = f16_bits(Stream(stream_seed(wid, TENSOR_SCALES))
                      .uniform_f16(groups * N, scale_lo, scale_hi).reshape(groups, N))
    zeros = None
    if not symmetric:
        zeros = Stream(stream_seed(wid, TENSOR_ZEROS)).nibbles(groups * N).reshape(groups, N)
    return codes, zeros, scales


def outlier_channels(K: int, count: int, wid: int) -> np.ndarray:
    """``count`` distinct channels of 0..K-1 by a partial Fisher-Yates shuffle."""
    perm = np.arange(K, dtype=np.int64)
    s = Stream(stream_seed(wid, TENSOR_OUTLIERS))
    for i in range(count):
        j = i + int(s.raw(1)[0] % np.uint64(K - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


def make_x(M: int, K: int, wid: int, n_outliers: int = 0, gain: float = 1.0) -> np.ndarray:
    """fp16 activations X[M][K] (uint16 bit patterns), ~N(0,1); ``n_outliers``
    channels (the same for every row) are multiplied by ``gain`` and re-rounded."""
    x = Stream(stream_seed(wid, TENSOR_X)).normal_f16(M * K).reshape(M, K)
    if n_outliers:
        ch = outlier_channels(K, n_outliers, wid)
        x[:, ch] = (x[:, ch].astype(np.float64) * gain).astype(np.float16)
    return f16_bits(x)


def workload_inputs(w: Workload, M: int | None = None):
    """(X, codes, zeros, scales) for workload ``w`` (X has ``M`` rows if given)."""
    codes, zeros, scales = make_layer(w.K, w.N, w.G, w.symmetric, w.scale_lo, w.scale_hi, w.wid)
    X = make_x(w.M if M is None else M, w.K, w.wid, w.n_outliers, w.outlier_gain)
    return X, codes, zeros, scales
