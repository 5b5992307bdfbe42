"""Cached inputs for the GPU parity tests.

Both sides start from the same synthetic arrays (``synth``): the oracle packs
and dequantizes them on the CPU, the HIP library packs them on the GPU.  Nothing
the GPU produces is ever fed to the oracle.
"""
from __future__ import annotations

import functools

import numpy as np

import oracle
from parity import to_dev
from w4a16_group_quantized_amd import binding, synth


@functools.lru_cache(maxsize=None)
def workload_host(name: str):
    """(X, codes, zeros, scales) for a named workload."""
    return synth.workload_inputs(synth.WORKLOADS[name])


@functools.lru_cache(maxsize=None)
def oracle_weight(name: str):
    """Oracle-side packed layer and dequantized W for a named workload."""
    w = synth.WORKLOADS[name]
    _, codes, zeros, scales = workload_host(name)
    o = oracle.load()
    Q = o.pack(codes)
    QZ = None if zeros is None else o.pack_zeros(zeros)
    W = o.dequant(Q, scales, QZ, w.G)
    return Q, QZ, W


_DEVICE_LAYERS = {}


def device_layer(name: str) -> binding.Layer:
    """The workload's layer packed on the GPU by the library."""
    if name not in _DEVICE_LAYERS:
        w = synth.WORKLOADS[name]
        _, codes, zeros, scales = workload_host(name)
        _DEVICE_LAYERS[name] = binding.make_layer(
            to_dev(codes), None if zeros is None else to_dev(zeros), to_dev(scales), w.G)
    return _DEVICE_LAYERS[name]


def random_case(seed: int, M: int, K: int, N: int, G: int, symmetric: bool,
                scale_lo: float = 0.002, scale_hi: float = 0.02):
    """Seeded inputs of an arbitrary shape (drawn by synth, with ``seed`` as the
    workload id)."""
    codes, zeros, scales = synth.make_layer(K, N, G, symmetric, scale_lo, scale_hi, seed)
    X = synth.make_x(M, K, seed)
    return X, codes, zeros, scales


def oracle_case(X, codes, zeros, scales, G, rows=None):
    o = oracle.load()
    Q = o.pack(codes)
    QZ = None if zeros is None else o.pack_zeros(zeros)
    W = o.dequant(Q, scales, QZ, G)
    Xs = X if rows is None else np.ascontiguousarray(X[rows])
    _, Y16 = o.matmul_w(Xs, W)
    return W, Y16


def device_case(codes, zeros, scales, G) -> binding.Layer:
    return binding.make_layer(to_dev(codes), None if zeros is None else to_dev(zeros),
                              to_dev(scales), G)
