"""Helpers for the GPU parity tests: moving synthetic inputs to the device and
the acceptance bar for the layer output.

The bar for Y (fp32 accumulation, fp16 out) against the oracle's fp16 result:
    max |Y - Y_ref| <= 1e-2 * max |Y_ref|   and   ||Y - Y_ref||_2 <= 2e-3 ||Y_ref||_2,
computed in double, and no non-finite Y where Y_ref is finite.  Packing and
dequantized weights are compared bit for bit.
"""
from __future__ import annotations

import numpy as np

MAX_REL = 1e-2
L2_REL = 2e-3


def h2f(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def to_dev(a: np.ndarray, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:        # fp16 bit patterns
        t = torch.from_numpy(a.view(np.int16)).view(torch.float16)
    elif a.dtype == np.int32:
        t = torch.from_numpy(a)
    elif a.dtype == np.uint8:
        t = torch.from_numpy(a)
    else:
        raise TypeError(a.dtype)
    return t.to("cuda")


def to_host_bits(t) -> np.ndarray:
    """Device fp16 tensor -> uint16 bit patterns."""
    import torch
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def y_errors(y_bits: np.ndarray, ref_bits: np.ndarray):
    y, r = h2f(y_bits), h2f(ref_bits)
    finite = np.isfinite(r)
    bad_nonfinite = int(np.sum(finite & ~np.isfinite(y)))
    d = np.abs(y - r)[finite]
    rmax = float(np.max(np.abs(r[finite]))) if finite.any() else 0.0
    max_rel = float(d.max()) / rmax if rmax > 0 else float(d.max())
    nr = float(np.linalg.norm(r[finite]))
    l2_rel = float(np.linalg.norm(d)) / nr if nr > 0 else float(np.linalg.norm(d))
    return max_rel, l2_rel, bad_nonfinite


def assert_y_close(y_bits: np.ndarray, ref_bits: np.ndarray, what: str = ""):
    assert y_bits.shape == ref_bits.shape, (y_bits.shape, ref_bits.shape)
    max_rel, l2_rel, bad = y_errors(y_bits, ref_bits)
    assert bad == 0, f"{what}: {bad} non-finite outputs where the oracle is finite"
    assert max_rel <= MAX_REL, f"{what}: max |dY| / max |Y_ref| = {max_rel:.3e} > {MAX_REL}"
    assert l2_rel <= L2_REL, f"{what}: relative L2 error {l2_rel:.3e} > {L2_REL}"
    return max_rel, l2_rel


def same_halves_up_to_zero_sign(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, dtype=np.uint16)
    b = np.asarray(b, dtype=np.uint16)
    za = (a & 0x7FFF) == 0
    zb = (b & 0x7FFF) == 0
    return bool(np.all((a == b) | (za & zb)))
