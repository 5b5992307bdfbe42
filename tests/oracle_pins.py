"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError if
the oracle disagrees with a value or property that does not come from the
oracle itself:

* hand-worked values stored under ``tests/golden/`` (each file states the
  passage of the pages it follows and shows the working);
* closed forms computed by hand (sums of arithmetic series, one-hot inputs,
  sign and power-of-two symmetries);
* numpy's own IEEE binary16 conversion, an implementation independent of the
  oracle's codec, as the library routine that the fp16 special cases reduce to;
* exact rational brute force (``fractions.Fraction``) on tiny layers, built
  from the *unpacked* inputs so that it shares no indexing with the oracle.

``tests/test_oracle_pins.py`` runs every pin against the oracle;
``tests/test_oracle_mutants.py`` compiles copies of ``oracle.c`` with a
plausible mistake planted and checks that some pin fails for each.
"""
from __future__ import annotations

import os
import sys
from fractions import Fraction

import math

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# helpers (numpy only; nothing from the oracle or the HIP library)
# ----------------------------------------------------------------------------

def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def _np_h2d(h):
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def _np_d2h(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def _same_halves(a, b):
    """Bitwise equality of fp16 patterns, NaNs compared by class."""
    a = np.asarray(a, dtype=np.uint16)
    b = np.asarray(b, dtype=np.uint16)
    nan_a = ((a & 0x7C00) == 0x7C00) & ((a & 0x03FF) != 0)
    nan_b = ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return bool(np.all((a == b) | (nan_a & nan_b)))


def _frac_to_half(q):
    """IEEE binary16 bits of the rational q rounded once, to nearest, ties to
    even (exact rational arithmetic; overflow to infinity at 65520)."""
    q = Fraction(q)
    sign = 0x8000 if q < 0 else 0
    a = -q if q < 0 else q
    if a == 0:
        return sign
    if a >= 65520:
        return sign | 0x7C00
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                               # now 2^e <= a < 2^(e+1)
    e = max(e, -14)                          # subnormals share the exponent -14
    m = a / Fraction(2) ** (e - 10)          # significand in units of the last place
    n = m.numerator // m.denominator
    rest = m - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n == 2048:                            # rounded up into the next binade
        n, e = 1024, e + 1
    if n < 1024:                             # subnormal
        return sign | n
    return sign | ((e + 15) << 10) | (n - 1024)


def _pack_by_hand(codes_col):
    """One word from eight codes, code j in bits 4j.. (for building inputs only)."""
    w = 0
    for j, c in enumerate(codes_col):
        w |= (int(c) & 0xF) << (4 * j)
    return w - (1 << 32) if w >= (1 << 31) else w


# ----------------------------------------------------------------------------
# fp16 codec: IEEE 754 binary16, checked against numpy's conversion
# ----------------------------------------------------------------------------

def pin_h2d_all_halves(o):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.h2d_array(h)
    want = _np_h2d(h)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_d2h_roundtrip_all_halves(o):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = _np_h2d(h)
    assert _same_halves(o.d2h_array(x), h)


def pin_d2h_midpoints(o):
    """Halfway cases tie to even; a hair either side rounds to the nearer half."""
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)  # +0 .. 65504
    lo = _np_h2d(h)
    hi = np.append(lo[1:], 65536.0)
    mid = (lo + hi) / 2.0           # exact in double
    for x in (mid, np.nextafter(mid, -np.inf), np.nextafter(mid, np.inf)):
        for sgn in (1.0, -1.0):
            assert _same_halves(o.d2h_array(sgn * x), _np_d2h(sgn * x))
    # the even neighbour wins every exact tie (65504 + 16 ties to 65536, infinity)
    even = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(o.d2h_array(mid), even)
    assert np.array_equal(o.d2h_array(np.nextafter(mid, -np.inf)), h)
    assert np.array_equal(o.d2h_array(np.nextafter(mid, np.inf)), (h + 1).astype(np.uint16))
    # the edges: the largest half, the overflow threshold, the smallest subnormal
    assert o.d2h(65504.0) == 0x7BFF
    assert o.d2h(np.nextafter(65520.0, 0.0)) == 0x7BFF
    assert o.d2h(65520.0) == 0x7C00
    assert o.d2h(2.0 ** -24) == 0x0001
    assert o.d2h(2.0 ** -25) == 0x0000            # tie between 0 and 2^-24 goes to 0
    assert o.d2h(3 * 2.0 ** -26) == 0x0001
    assert o.d2h(-0.0) == 0x8000
    assert o.d2h(float("inf")) == 0x7C00 and o.d2h(float("-inf")) == 0xFC00
    assert (o.d2h(float("nan")) & 0x7C00) == 0x7C00 and (o.d2h(float("nan")) & 0x3FF) != 0


def pin_d2h_random(o):
    rng = np.random.default_rng(12345)
    x = rng.standard_normal(400_000) * np.exp2(rng.integers(-30, 18, 400_000))
    assert _same_halves(o.d2h_array(x), _np_d2h(x))


# ----------------------------------------------------------------------------
# packing: eight 4-bit codes per 32-bit word
# ----------------------------------------------------------------------------

def _golden_pack():
    codes, words = [], []
    for f in _rows("pack_words.txt"):
        codes.append([int(c) for c in f[0].split(",")])
        words.append(int(f[2]))
        assert (int(f[1], 16) - (1 << 32) if int(f[1], 16) >= 1 << 31 else int(f[1], 16)) == int(f[2])
    return codes, words


def pin_pack_golden(o):
    codes, words = _golden_pack()
    ncol = len(codes)
    npad = (ncol + 7) // 8 * 8
    C = np.zeros((8, npad), dtype=np.uint8)
    for n, col in enumerate(codes):
        C[:, n] = col
    Q = o.pack(C)
    assert Q.shape == (1, npad)
    assert [int(v) for v in Q[0, :ncol]] == words
    # the same words unpack to the codes' low nibbles, in order
    back = o.unpack(Q)
    for n, col in enumerate(codes):
        assert [int(v) for v in back[:, n]] == [c & 0xF for c in col]


def pin_pack_zeros_golden(o):
    """Zero points pack eight consecutive columns into one word, column j in bits 4j."""
    codes, words = _golden_pack()
    Z = np.array(codes, dtype=np.uint8).reshape(len(codes), 8)  # groups x 8 columns
    QZ = o.pack_zeros(Z)
    assert QZ.shape == (len(codes), 1)
    assert [int(v) for v in QZ[:, 0]] == words
    assert np.array_equal(o.unpack_zeros(QZ), Z & 0xF)


def pin_pack_roundtrip(o):
    rng = np.random.default_rng(7)
    c = rng.integers(0, 256, size=(64, 40), dtype=np.uint8)
    Q = o.pack(c)
    assert Q.shape == (8, 40)
    assert np.array_equal(o.unpack(Q), c & 0xF)
    # packing is a bijection on words: every 32-bit pattern comes back
    w = rng.integers(-(1 << 31), 1 << 31, size=(5, 48), dtype=np.int64).astype(np.int32)
    assert np.array_equal(o.pack(o.unpack(w)), w)
    assert np.array_equal(o.pack_zeros(o.unpack_zeros(w)), w)
    # a code written at (k, n) by hand is found at (k, n)
    for k, n in [(0, 0), (7, 3), (13, 39), (63, 1)]:
        cc = np.zeros((64, 40), dtype=np.uint8)
        cc[k, n] = 11
        Qh = np.zeros((8, 40), dtype=np.int32)
        Qh[k // 8, n] = _pack_by_hand([11 if j == k % 8 else 0 for j in range(8)])
        assert np.array_equal(o.pack(cc), Qh)


def pin_packed_size(o):
    """qweight is four times smaller than the fp16 weight (8 codes per 4 bytes)."""
    for K, N in [(8, 8), (128, 64), (512, 512)]:
        Q = o.pack(np.zeros((K, N), dtype=np.uint8))
        assert Q.nbytes == K * N // 2 and 2 * K * N == 4 * Q.nbytes


def pin_interleave_golden(o):
    """Hand-worked interleaved words (tests/golden/interleave_words.txt), from
    the unpacked codes of one column; and back."""
    for codes, canon, inter in _rows("interleave_words.txt"):
        col = np.array([int(c) for c in codes.split(",")], dtype=np.uint8)
        Q = o.pack(col[:, None])
        assert int(np.uint32(Q[0, 0])) == int(canon, 16), codes
        I = o.interleave(Q)
        assert int(np.uint32(I[0, 0])) == int(inter, 16), (codes, hex(int(np.uint32(I[0, 0]))))
        assert np.array_equal(o.deinterleave(I), Q)


def pin_interleave_positions_and_round_trip(o):
    """On random codes, code k of the interleaved word [k/8][n] is the nibble at
    bit 4 (4 (k % 2) + (k % 8) / 2), read with Python integers from the
    unpacked codes; deinterleave undoes interleave and interleave undoes
    deinterleave on arbitrary 32-bit words (a permutation of nibbles)."""
    rng = np.random.default_rng(35)
    K, N = 64, 24
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    I = o.interleave(o.pack(codes)).view(np.uint32)
    for k in range(K):
        for n in range(0, N, 5):
            pos = 4 * (k % 2) + (k % 8) // 2
            assert (int(I[k // 8, n]) >> (4 * pos)) & 0xF == codes[k, n], (k, n)
    W = rng.integers(-(1 << 31), 1 << 31, (16, 40), dtype=np.int64).astype(np.int32)
    assert np.array_equal(o.deinterleave(o.interleave(W)), W)
    assert np.array_equal(o.interleave(o.deinterleave(W)), W)
    assert not np.array_equal(o.interleave(W), W)


def pin_block_hand_worked(o):
    """The blocked layout's places, worked by hand from its definition for
    K = 16 (two packed rows) and N = 256 (two blocks), word (r, n) = 1000 r + n:
    block 0 holds row 0 then row 1 of columns 0..127, block 1 the same for
    columns 128..255."""
    Q = (1000 * np.arange(2)[:, None] + np.arange(256)[None, :]).astype(np.int32)
    B = o.block(Q)
    want = {0: 0, 1: 1, 127: 127, 128: 1000, 129: 1001, 255: 1127,
            256: 128, 383: 255, 384: 1128, 511: 1255}
    for i, v in want.items():
        assert int(B[i]) == v, (i, int(B[i]), v)
    assert np.array_equal(o.unblock(B, 16, 256), Q)


def pin_block_strips_and_round_trip(o):
    """Each 128-column strip of the words is one contiguous run, its rows in
    order (numpy slicing of the logical array); unblock undoes block; with one
    block or one packed row the words do not move; the words are only moved
    (same multiset)."""
    rng = np.random.default_rng(36)
    for K, N in ((64, 384), (8, 512), (1024, 128), (24, 1280)):
        Q = rng.integers(-(1 << 31), 1 << 31, (K // 8, N), dtype=np.int64).astype(np.int32)
        B = o.block(Q)
        R = K // 8
        for b in range(N // 128):
            run = B[b * R * 128:(b + 1) * R * 128].reshape(R, 128)
            assert np.array_equal(run, Q[:, 128 * b:128 * (b + 1)]), (K, N, b)
        assert np.array_equal(o.unblock(B, K, N), Q)
        assert np.array_equal(np.sort(B), np.sort(Q.reshape(-1)))
        if N == 128 or R == 1:
            assert np.array_equal(B, Q.reshape(-1))
        else:
            assert not np.array_equal(B, Q.reshape(-1))


# ----------------------------------------------------------------------------
# dequantization w = fp16(s * (q - z))
# ----------------------------------------------------------------------------

def pin_dequant_golden(o):
    for f in _rows("dequant_examples.txt"):
        q, z, s, w = int(f[0]), int(f[1]), int(f[2], 16), int(f[3], 16)
        assert o.dequant_one(q, z, s) == w, (q, z, hex(s))
        assert float(np.uint16(w).view(np.float16)) == float(f[4])
        # the same example through the tensor path: one column, one group of 8
        codes = np.full((8, 8), q, dtype=np.uint8)
        zeros = np.full((1, 8), z, dtype=np.uint8)
        S = np.full((1, 8), s, dtype=np.uint16)
        W = o.dequant(o.pack(codes), S, o.pack_zeros(zeros), 8)
        assert np.all(W == w)


def pin_dequant_exhaustive(o):
    """Every code, every zero and every finite fp16 scale, through the tensor path.

    Layout: group g (G = 16) carries zero point g; inside it, row k carries code
    k % 16; column n carries the n-th finite fp16 pattern as its scale in every
    group.  The reference is numpy's rounding of the exact double product.
    """
    all_h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = all_h[(all_h & 0x7C00) != 0x7C00]          # 63488 patterns
    N = finite.size
    G, groups = 16, 16
    K = G * groups
    codes = np.tile((np.arange(K) % 16).astype(np.uint8)[:, None], (1, N))
    zeros = np.tile(np.arange(groups, dtype=np.uint8)[:, None], (1, N))
    S = np.tile(finite[None, :], (groups, 1))
    W = o.dequant(o.pack(codes), S, o.pack_zeros(zeros), G)
    s64 = _np_h2d(finite)
    diff = (np.arange(K) % 16 - np.arange(K) // 16).astype(np.float64)
    want = _np_d2h(diff[:, None] * s64[None, :])
    assert _same_halves(W, want)
    # symmetric: no zero tensor means z = 8
    Ws = o.dequant(o.pack(codes[:16]), S[:1], None, 16)
    wants = _np_d2h((np.arange(16) - 8).astype(np.float64)[:, None] * s64[None, :])
    assert _same_halves(Ws, wants)


def pin_dequant_invariants(o):
    s_vals = [0x211F, 0x1419, 0x251F, 0x3C00, 0x0001, 0x7BFF]
    for s in s_vals:
        sv = float(np.uint16(s).view(np.float16))
        for q in range(16):
            assert o.dequant_one(q, q, s) == 0x0000          # q == z gives +0 for s > 0
        assert o.dequant_one(8, 8, s) == 0x0000               # symmetric code 8 -> 0
        assert o.dequant_one(0, 8, s) == int(_np_d2h(-8 * sv))  # code 0 -> -8s
        assert o.dequant_one(15, 8, s) == int(_np_d2h(7 * sv))  # code 15 -> 7s
        # (q - z) and (z - q) give results of opposite sign and equal magnitude
        for q, z in [(3, 8), (15, 0), (1, 2)]:
            assert o.dequant_one(q, z, s) ^ o.dequant_one(z, q, s) == 0x8000


# ----------------------------------------------------------------------------
# the layer Y = X @ W
# ----------------------------------------------------------------------------

def pin_tiny_gemv_golden(o):
    codes = np.array([[(k + n) % 16 for n in range(8)] for k in range(8)], dtype=np.uint8)
    Q = o.pack(codes)
    assert [int(v) & 0xFFFFFFFF for v in Q[0]] == [0x76543210 + n * 0x11111111 for n in range(8)]
    X = np.full((1, 8), 0x3C00, dtype=np.uint16)    # ones
    for f in _rows("tiny_gemv.txt"):
        s = int(f[1], 16)
        QZ = None if f[2] == "none" else o.pack_zeros(
            np.array([[int(v) for v in f[2].split(",")]], dtype=np.uint8))
        S = np.full((1, 8), s, dtype=np.uint16)
        Y64, Y16 = o.linear(X, Q, S, QZ, 8)
        want = [float(v) for v in f[3].split(",")]
        assert list(Y64[0]) == want, f[0]
        assert list(_np_h2d(Y16[0])) == want, f[0]


def pin_group_axis(o):
    """Groups run along K: with q - z = 1, group 0 scaled by 1 and group 1 by 2,
    rows 0..7 of W are 1 and rows 8..15 are 2 in every column."""
    K, N, G = 16, 8, 8
    Q = o.pack(np.full((K, N), 9, dtype=np.uint8))
    QZ = o.pack_zeros(np.full((2, N), 8, dtype=np.uint8))
    S = np.array([[0x3C00] * N, [0x4000] * N], dtype=np.uint16)   # 1.0, 2.0
    one = 0x3C00
    for x, want in [([one] * 16, 24.0), ([one] * 8 + [0] * 8, 8.0), ([0] * 8 + [one] * 8, 16.0),
                    ([0] * 15 + [one], 2.0)]:
        Y64, _ = o.linear(np.array([x], dtype=np.uint16), Q, S, QZ, G)
        assert np.all(Y64 == want), (x, Y64)


def pin_scale_and_zero_columns(o):
    """Scales and zeros are per column: s[n] = n + 1 and z[n] = 8 - (n % 3) with
    code 9 give W[k][n] = (n + 1) * (1 + n % 3)."""
    K, N, G = 8, 16, 8
    Q = o.pack(np.full((K, N), 9, dtype=np.uint8))
    zeros = np.array([[8 - (n % 3) for n in range(N)]], dtype=np.uint8)
    S = _np_d2h(np.arange(1, N + 1, dtype=np.float64))[None, :]
    X = np.zeros((1, K), dtype=np.uint16)
    X[0, 3] = 0x3C00
    Y64, Y16 = o.linear(X, Q, S, o.pack_zeros(zeros), G)
    assert list(Y64[0]) == [float((n + 1) * (1 + n % 3)) for n in range(N)]


def pin_onehot(o):
    """X = e_k returns row k of the dequantized weight bit for bit."""
    rng = np.random.default_rng(3)
    K, N, G = 64, 24, 16
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    S = _np_d2h(rng.uniform(0.002, 0.02, (K // G, N)))
    Q, QZ = o.pack(codes), o.pack_zeros(zeros)
    W = o.dequant(Q, S, QZ, G)
    X = np.zeros((K, K), dtype=np.uint16)
    X[np.arange(K), np.arange(K)] = 0x3C00                  # identity: row m = e_m
    _, Y16 = o.linear(X, Q, S, QZ, G)
    assert _same_halves(Y16, W)


def _exact_layer(X, codes, zeros, S, G):
    """Exact rational Y from unpacked inputs: w = fp16(s (q - z)) rounded by numpy,
    then sum of exact products."""
    M, K = X.shape
    N = codes.shape[1]
    xs = [[Fraction(float(v)) for v in row] for row in _np_h2d(X)]
    W = np.empty((K, N), dtype=np.float64)
    for k in range(K):
        g = k // G
        for n in range(N):
            z = 8 if zeros is None else int(zeros[g, n])
            W[k, n] = _np_h2d(_np_d2h((int(codes[k, n]) - z) * float(_np_h2d(S[g, n]))))
    ws = [[Fraction(float(v)) for v in row] for row in W]
    exact = [[sum((xs[m][k] * ws[k][n] for k in range(K)), Fraction(0)) for n in range(N)]
             for m in range(M)]
    absum = [[sum((abs(xs[m][k] * ws[k][n]) for k in range(K)), Fraction(0)) for n in range(N)]
             for m in range(M)]
    return exact, absum


def pin_bruteforce_exact(o):
    rng = np.random.default_rng(11)
    for M, K, N, G, sym in [(1, 8, 8, 8, False), (3, 16, 24, 8, False), (2, 128, 16, 128, False),
                            (3, 256, 8, 128, True), (1, 64, 16, 64, True), (16, 32, 8, 16, False)]:
        codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
        zeros = None if sym else rng.integers(0, 16, (K // G, N), dtype=np.uint8)
        S = _np_d2h(rng.uniform(0.002, 0.02, (K // G, N)))
        X = _np_d2h(rng.standard_normal((M, K)))
        Y64, Y16 = o.linear(X, o.pack(codes), S, None if sym else o.pack_zeros(zeros), G)
        exact, absum = _exact_layer(X, codes, zeros, S, G)
        for m in range(M):
            for n in range(N):
                e = exact[m][n]
                # recursive summation in double: |error| <= (K - 1) u sum|terms|, u = 2^-53
                assert abs(Fraction(Y64[m, n]) - e) <= K * Fraction(1, 1 << 53) * absum[m][n]
                assert int(Y16[m, n]) == int(_np_d2h(float(e))), (M, K, N, m, n)


def pin_power_of_two(o):
    """Doubling X or the scales doubles Y exactly (no overflow or underflow here)."""
    rng = np.random.default_rng(5)
    K, N, G = 256, 32, 128
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    zeros = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    S = _np_d2h(rng.uniform(0.002, 0.02, (K // G, N)))
    X = _np_d2h(rng.standard_normal((4, K)))
    Q, QZ = o.pack(codes), o.pack_zeros(zeros)
    Y64, Y16 = o.linear(X, Q, S, QZ, G)
    Y64x, Y16x = o.linear(_np_d2h(2.0 * _np_h2d(X)), Q, S, QZ, G)
    Y64s, Y16s = o.linear(X, Q, _np_d2h(4.0 * _np_h2d(S)), QZ, G)
    assert np.array_equal(Y64x, 2.0 * Y64) and np.array_equal(Y64s, 4.0 * Y64)
    assert np.array_equal(_np_h2d(Y16x), 2.0 * _np_h2d(Y16))
    assert np.array_equal(_np_h2d(Y16s), 4.0 * _np_h2d(Y16))
    # negating X negates Y
    Yn64, _ = o.linear(X ^ np.uint16(0x8000), Q, S, QZ, G)
    assert np.array_equal(Yn64, -Y64)


def pin_rows_independent(o):
    """Each output row depends on its own X row only (sampled parity relies on it)."""
    rng = np.random.default_rng(9)
    K, N, G = 128, 40, 32
    codes = rng.integers(0, 16, (K, N), dtype=np.uint8)
    S = _np_d2h(rng.uniform(0.002, 0.02, (K // G, N)))
    X = _np_d2h(rng.standard_normal((6, K)))
    Q = o.pack(codes)
    Y64, Y16 = o.linear(X, Q, S, None, G)
    rows = [4, 1]
    Y64r, Y16r = o.linear(X[rows], Q, S, None, G)
    assert np.array_equal(Y64r, Y64[rows]) and np.array_equal(Y16r, Y16[rows])


def _lambert_w_inv_e():
    """W(1/e): the root of w e^w = 1/e, by Newton's method in plain floats."""
    w = 0.25
    for _ in range(60):
        f = w * math.exp(w) - math.exp(-1.0)
        w -= f / (math.exp(w) * (w + 1.0))
    return w


def pin_silu_closed_forms(o):
    """SiLU(t) = t sigmoid(t): values the definition fixes in closed form."""
    ln3 = math.log(3.0)
    assert o.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4
    assert abs(o.silu(ln3) - 0.75 * ln3) <= 4e-16 * ln3
    assert abs(o.silu(-ln3) + 0.25 * ln3) <= 4e-16 * ln3
    # sigmoid(t) + sigmoid(-t) = 1, hence SiLU(t) - SiLU(-t) = t
    rng = np.random.default_rng(21)
    for t in rng.uniform(-30.0, 30.0, 200):
        assert abs(o.silu(t) - o.silu(-t) - t) <= 1e-14 * max(1.0, abs(t))
    # saturation: SiLU(t) = t once e^-t is below half an ulp of 1; tiny and
    # negative far below zero, and the correctly signed zero past overflow
    assert o.silu(60.0) == 60.0
    assert -1e-24 < o.silu(-60.0) < 0.0
    assert o.silu(-800.0) == 0.0 and math.copysign(1.0, o.silu(-800.0)) < 0
    # the global minimum: at t* = -1 - W(1/e), SiLU(t*) = t* + 1 = -W(1/e)
    w = _lambert_w_inv_e()
    t_star = -1.0 - w
    assert abs(o.silu(t_star) + w) <= 1e-15
    grid = np.linspace(t_star - 0.01, t_star + 0.01, 2001)
    assert min(o.silu(t) for t in grid) >= -w - 1e-15


def pin_gate_up_composition(o):
    """Fused gate/up on a hand-built layer: columns [gate | up], h = SiLU(gate) up.

    K = G = 8, X = ones (twos in row 2), s = 1, z = 0, so each output is its
    column's code sum (doubled in row 2).  Gate sums of 0 give h = 0 whatever
    the up column; gate sums of 16 and 32 saturate SiLU to within 1.2e-7
    relative, so h = fp16(gate * up) there; gate sums from 1 to 10 are where
    SiLU bends: there sigmoid(t) = e^t / (1 + e^t), evaluated with the constant
    e, and h is that times t and up, rounded to fp16 (numpy's conversion).
    N = 2I = 32 keeps whole words of packed zero points.
    """
    I = 16
    gate = [0, 16, 16, 0, 16, 0, 16, 16, 1, 2, 3, 5, 1, 0, 2, 16]
    up = [40, 3, 0, 120, 1, 8, 6, 2, 7, 9, 11, 5, 30, 4, 13, 0]
    codes = np.zeros((8, 2 * I), dtype=np.uint8)
    for n in range(I):
        for c, total in ((n, gate[n]), (I + n, up[n])):
            left = total
            for k in range(8):          # spread each sum over the 8 codes
                codes[k, c] = min(15, left)
                left -= codes[k, c]
            assert left == 0
    Q = o.pack(codes)
    S = np.full((1, 2 * I), 0x3C00, dtype=np.uint16)
    QZ = o.pack_zeros(np.zeros((1, 2 * I), dtype=np.uint8))
    X = np.array([[0x3C00] * 8, [0x4000] * 8], dtype=np.uint16)   # ones, twos
    Y64, _ = o.linear(X, Q, S, QZ, 8)
    assert list(Y64[0, :I]) == gate and list(Y64[0, I:]) == up
    H = o.gate_up(Y64)

    def sig(t):
        return math.e ** t / (1.0 + math.e ** t)

    for row, f in ((0, 1), (1, 2)):
        for n in range(I):
            g, u = f * gate[n], f * up[n]
            if g == 0:
                want = 0.0
            elif g >= 16:
                want = float(g * u)
            else:
                want = g * sig(g) * u
            assert H[row, n] == _np_d2h(np.array([want]))[0], (row, n, _np_h2d(H[row, n]), want)


def _grid_layer(rng, K, N, G, symmetric):
    """Weights that are exactly s (q - z) on a per-group grid with power-of-two
    scales (exact in fp16), every group reaching both ends of its range."""
    groups = K // G
    # symmetric: s = max|w| / 7 maps the grid to codes 1..15 (-7 s .. 7 s)
    codes = rng.integers(1 if symmetric else 0, 16, (K, N)).astype(np.uint8)
    exps = rng.integers(-12, -2, (groups, N))
    S = np.ldexp(1.0, exps)
    if symmetric:
        Z = np.full((groups, N), 8)
        ends = (1, 15)                       # +-7 s: the symmetric scale is max|w| / 7
    else:
        Z = rng.integers(0, 16, (groups, N))
        ends = (0, 15)
    for g in range(groups):
        codes[g * G, :] = ends[0]
        codes[g * G + 1, :] = ends[1]
    Zk = np.repeat(Z, G, axis=0)
    Sk = np.repeat(S, G, axis=0)
    W = (codes.astype(np.float64) - Zk) * Sk
    return _np_d2h(W), codes, _np_d2h(S), Z.astype(np.uint8)


def pin_quantize_recovers_grid(o):
    """Min-max over a group spanning its whole grid recovers that grid exactly:
    lo = -z s and hi = (15 - z) s give s = range / 15 and z = -lo / s."""
    rng = np.random.default_rng(31)
    for sym in (False, True):
        W, codes, S, Z = _grid_layer(rng, 256, 24, 64, sym)
        c2, S2, Z2 = o.quantize(W, 64, sym)
        assert np.array_equal(S2, S), sym
        assert np.array_equal(c2, codes), sym
        if not sym:
            assert np.array_equal(Z2, Z)


def pin_quantize_nearest_code(o):
    """Given its scale and zero point, every code is the nearest of the 16 levels
    (brute force over all codes), and the scale is range / 15 (or max|w| / 7)
    rounded once to fp16."""
    rng = np.random.default_rng(32)
    K, N, G = 64, 12, 16
    for sym in (False, True):
        W = _np_d2h(rng.standard_normal((K, N)) * rng.uniform(0.001, 0.1, (1, N)))
        codes, S, Z = o.quantize(W, G, sym)
        w = _np_h2d(W)
        for g in range(K // G):
            blk = w[g * G:(g + 1) * G]
            for n in range(N):
                col = [Fraction(float(v)) for v in blk[:, n]]
                r = (max(col) - min(col)) / 15 if not sym else max(abs(v) for v in col) / 7
                assert int(S[g][n]) == _frac_to_half(r), (sym, g, n)
            s = _np_h2d(S[g])
            z = np.full(N, 8) if sym else Z[g].astype(np.int64)
            levels = (np.arange(16)[:, None] - z[None, :]) * s[None, :]      # [16][N]
            for k in range(g * G, (g + 1) * G):
                err = np.abs(w[k][None, :] - levels)                            # [16][N]
                best = err.min(0)
                got = err[codes[k], np.arange(N)]
                assert np.all(got <= best * (1 + 1e-6) + 1e-12), (sym, k)


def _scale_groups(o, pairs, symmetric):
    """Quantize one 8-row group per column whose extremes are the given fp16
    (hi, lo) pairs (the other rows lie between them); return the scales."""
    pairs = list(pairs)
    N = -(-len(pairs) // 8) * 8
    hi = np.full(N, 0x3C00, dtype=np.uint16)
    lo = np.full(N, 0xBC00, dtype=np.uint16)
    for i, (h, l) in enumerate(pairs):
        hi[i], lo[i] = h, l
    W = np.empty((8, N), dtype=np.uint16)
    W[0], W[1:] = hi, lo
    _, S, _ = o.quantize(W, 8, symmetric)
    return S[0][:len(pairs)]


def pin_quantize_scale_exact(o):
    """The scale is the exact (hi - lo) / 15 (or max|w| / 7) rounded once to
    fp16, checked with rational arithmetic.  The fp16 extremes hi = 693.5,
    lo = -0.015594482421875 give (hi - lo) / 15 = 46.2343729..., which rounds
    to 46.21875 (0x51C7); forming hi - lo in fp32 first lands on a tie and
    gives 46.25 (0x51C8).  More such groups come from a seeded search over
    random fp16 extremes for pairs where an fp32 range or quotient would
    round differently; their expected scales are computed exactly here.
    Symmetric: every positive finite fp16 max|w|, exhaustively."""
    h = lambda v: int(np.float16(v).view(np.uint16))
    want = _frac_to_half((Fraction(693.5) + Fraction(0.015594482421875)) / 15)
    assert want == 0x51C7
    S = _scale_groups(o, [(h(693.5), h(-0.015594482421875))], False)
    assert int(S[0]) == 0x51C7, hex(int(S[0]))

    rng = np.random.default_rng(34)
    a = rng.integers(0, 0x7C00, 1 << 21).astype(np.uint16)
    b = rng.integers(0, 0x7C00, 1 << 21).astype(np.uint16) | np.uint16(0x8000)
    fa = a.view(np.float16).astype(np.float32)
    fb = b.view(np.float16).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        f32 = ((fa - fb) / np.float32(15)).astype(np.float16).view(np.uint16)
        f64 = ((fa.astype(np.float64) - fb) / 15.0).astype(np.float16).view(np.uint16)
    # candidates only: the expected value of each is the exact one below
    cand = np.nonzero((f32 != f64) & np.isfinite(fa - fb))[0][:48]
    pairs = []
    for i in cand:
        exact = _frac_to_half((Fraction(float(fa[i])) - Fraction(float(fb[i]))) / 15)
        if exact != int(f32[i]):
            pairs.append((int(a[i]), int(b[i]), exact))
    assert len(pairs) >= 8, len(pairs)
    # and a plain sample of ordinary pairs
    for i in range(200):
        exact = _frac_to_half((Fraction(float(fa[i])) - Fraction(float(fb[i]))) / 15)
        pairs.append((int(a[i]), int(b[i]), exact))
    S = _scale_groups(o, [(p[0], p[1]) for p in pairs], False)
    for (hh, ll, exact), got in zip(pairs, S):
        want = exact if exact & 0x7FFF else 0x3C00
        assert int(got) == want, (hex(hh), hex(ll), hex(int(got)), hex(want))

    amax = np.arange(1, 0x7C00, dtype=np.uint16)
    S = _scale_groups(o, [(int(v), 0) for v in amax], True)
    for v, got in zip(amax, S):
        exact = _frac_to_half(Fraction(float(np.uint16(v).view(np.float16))) / 7)
        want = exact if exact & 0x7FFF else 0x3C00
        assert int(got) == want, (hex(int(v)), hex(int(got)), hex(want))


def pin_quantize_round_trip_bound(o):
    """|w - dequant(quantize(w))| <= s / 2 (plus the fp16 rounding of the
    dequantized weight) wherever the code is not clamped, and <= s at a clamp."""
    rng = np.random.default_rng(33)
    K, N, G = 512, 40, 128
    for sym in (False, True):
        W = _np_d2h(rng.standard_normal((K, N)) * 0.02)
        codes, S, Z = o.quantize(W, G, sym)
        QZ = None if sym else o.pack_zeros(Z)
        Wq = _np_h2d(o.dequant(o.pack(codes), S, QZ, G))
        w = _np_h2d(W)
        s = np.repeat(_np_h2d(S), G, axis=0)
        err = np.abs(w - Wq)
        slack = 2.0 ** -11 * np.abs(Wq) + 1e-12
        clamped = (codes == 0) | (codes == 15)
        assert np.all(err[~clamped] <= s[~clamped] / 2 + slack[~clamped]), sym
        assert np.all(err <= s + slack), sym


def pin_quantize_degenerate_groups(o):
    """A constant group c is reproduced (range |c|); an all-zero group gives
    codes equal to the zero point, scale 1."""
    K, N, G = 32, 8, 16
    c = np.array([0.5, -0.25, 3.0, -7.0, 0.0, 0.0, 1e-3, -2.0])
    W = _np_d2h(np.repeat(c[None, :], K, axis=0))
    for sym in (False, True):
        codes, S, Z = o.quantize(W, G, sym)
        QZ = None if sym else o.pack_zeros(Z)
        Wq = _np_h2d(o.dequant(o.pack(codes), S, QZ, G))
        w = _np_h2d(W)
        assert np.all(np.abs(Wq - w) <= 2.0 ** -9 * np.abs(w)), (sym, Wq[0], w[0])
        assert np.all(_np_h2d(S[:, 4]) == 1.0) and np.all(_np_h2d(S[:, 5]) == 1.0)


# --- scale migration and its search (R14, R15, R16) -----------------------

def pin_channel_stats_hand_worked(o):
    """A 2 x 8 X and an 8 x 2 W with G = 4, worked by hand: xbar is the mean
    |x| per channel; wbar the mean over columns of |w| over its group's max |w|
    (an all-zero group contributes 0)."""
    X = _np_d2h(np.array([[1, -2, 0.5, 4, -1, 0, 3, -0.25],
                          [-3, 2, 0.5, -4, 1, 0, -1, 0.75]], dtype=np.float64))
    W = _np_d2h(np.array([[1, -8], [-2, 8], [4, 2], [0, 1],
                          [0, 0.5], [0, -0.5], [0, 0.25], [0, 1]], dtype=np.float64))
    xbar, wbar = o.channel_stats(X, W, 4)
    assert list(xbar) == [2, 2, 0.5, 4, 1, 0, 2, 0.5]
    assert list(wbar) == [0.625, 0.75, 0.625, 0.0625, 0.25, 0.25, 0.125, 0.5]


def pin_scale_candidate_closed_forms(o):
    """alpha = 1 gives xbar, alpha = 0 gives 1 / wbar, alpha = 1/2 gives
    sqrt(xbar / wbar); statistics below 1e-4 count as 1e-4."""
    xbar = np.array([4.0, 0.25, 1e-6, 2.0])
    wbar = np.array([0.5, 1.0, 0.5, 1e-8])
    assert list(o.scale_candidate(xbar, wbar, 1.0)) == [4.0, 0.25, 1e-4, 2.0]
    assert list(o.scale_candidate(xbar, wbar, 0.0)) == [2.0, 1.0, 2.0, 1e4]
    half = o.scale_candidate(xbar, wbar, 0.5)
    want = [math.sqrt(4.0 / 0.5), math.sqrt(0.25), math.sqrt(1e-4 / 0.5), math.sqrt(2.0 / 1e-4)]
    assert all(abs(a - b) <= 1e-15 * b for a, b in zip(half, want)), (half, want)


def _dyadic_x(rng, M, K):
    """X = +-j / 8, j = 1..16: few significant bits, so products with grid
    weights and their sums are exact in fp64 in any order."""
    return _np_d2h(rng.integers(1, 17, (M, K)) / 8.0 * rng.choice([-1.0, 1.0], (M, K)))


def pin_migration_invariance_exact(o):
    """With c a power of two per channel and no value leaving the normal fp16
    range, X / c and c W are exact, so (X / c)(c W) = X W bit for bit: the
    migration is invisible before rounding."""
    rng = np.random.default_rng(41)
    M, K, N = 6, 64, 24
    X = _np_d2h(rng.uniform(2.0 ** -4, 4.0, (M, K)) * rng.choice([-1.0, 1.0], (M, K)))
    W = _np_d2h(rng.uniform(2.0 ** -8, 1.0, (K, N)) * rng.choice([-1.0, 1.0], (K, N)))
    c = np.ldexp(1.0, rng.integers(-3, 4, K))
    Xs, Ws = o.migrate(X, W, c)
    assert np.array_equal(_np_h2d(Xs), _np_h2d(X) / c)
    assert np.array_equal(_np_h2d(Ws), c[:, None] * _np_h2d(W))
    Y, _ = o.matmul_w(X, W)
    Ys, _ = o.matmul_w(Xs, Ws)
    assert np.array_equal(Y, Ys)


def pin_scale_loss_on_a_grid(o):
    """A weight already on each group's grid, scaled by a power of two constant
    within each group, stays on a grid that the quantizer recovers exactly; with
    X / c exact too, the candidate's output is fp16(X W) and the loss is the
    output rounding alone: mean((y - fp16(y))^2), with y computed in numpy."""
    rng = np.random.default_rng(42)
    M, K, N, G = 5, 256, 24, 64
    for sym in (False, True):
        W, _, _, _ = _grid_layer(rng, K, N, G, sym)
        X = _dyadic_x(rng, M, K)
        c = np.repeat(np.ldexp(1.0, rng.integers(-2, 3, K // G)), G)
        y = _np_h2d(X) @ _np_h2d(W)
        want = np.mean((y - _np_h2d(_np_d2h(y))) ** 2)
        assert want > 0.0
        assert o.scale_loss(X, W, G, sym, c) == want, sym
        # the same layer with c varying inside the groups leaves the grid
        c2 = np.ldexp(1.0, rng.integers(-2, 3, K))
        assert o.scale_loss(X, W, G, sym, c2) > want, sym


def pin_scale_search_first_minimum(o):
    """|x| = 1 everywhere and |w| constant within each group and column give
    xbar = wbar = 1, hence c = 1 for every alpha: all losses are equal, equal to
    the loss at c = 1, and the search keeps the first grid value."""
    rng = np.random.default_rng(43)
    M, K, N, G = 4, 128, 16, 32
    X = _np_d2h(rng.choice([-1.0, 1.0], (M, K)))
    a = np.repeat(np.ldexp(1.0, rng.integers(-8, -2, (K // G, N))), G, axis=0)
    W = _np_d2h(a * rng.choice([-1.0, 1.0], (K, N)))
    xbar, wbar = o.channel_stats(X, W, G)
    assert np.all(xbar == 1.0) and np.all(wbar == 1.0)
    alphas = [0.0, 0.3, 0.5, 0.9, 1.0]
    best, losses, cb = o.scale_search(X, W, G, False, alphas)
    assert best == 0
    assert np.all(losses == o.scale_loss(X, W, G, False, np.ones(K)))
    assert np.all(cb == 1.0)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def run_all(library_path):
    """Run every pin against the oracle library at ``library_path``; used by the
    mutation test in a child process (a planted mistake may crash)."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import oracle
    o = oracle.Oracle(library_path)
    failed = []
    for pin in PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    return failed


if __name__ == "__main__":
    bad = run_all(sys.argv[1])
    print("FAILED:" + ",".join(bad))
    sys.exit(1 if bad else 0)
