"""Plain CPU oracle for the W4A16 group-quantized linear layer (AWQ inference).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the repository's smoke check and
the CPU-baseline leg of ``bench.py`` may import this package.  The HIP library
and its Python binding never import, link or call anything here, and nothing
here imports them.

The arithmetic lives in ``oracle.c`` (plain C, single threaded, fp64
accumulation); this module only compiles it with gcc and wraps it for numpy.
Readings of the pages that the oracle follows are listed at the top of
``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

# Strict IEEE double arithmetic: no fast-math, no contraction into FMA.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off"]


def build(source: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile ``source`` with gcc into the shared library ``out``.  The object is
    written under a name of this process's own and renamed into place, so that
    processes building at once (parallel test workers) never share a file."""
    include = os.path.dirname(os.path.abspath(SOURCE))
    tmp = f"{out}.tmp{os.getpid():x}"
    cmd = ["gcc", *CFLAGS, "-I", include, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctype)


def _check_layer(K: int, N: int, G: int, S: np.ndarray, QZ) -> None:
    """Shapes the packed layout fixes: eight codes per qweight word along K,
    eight zero points per qzeros word along N, one scale row per group of G."""
    if G <= 0 or K % G != 0:
        raise ValueError(f"group size {G} must divide K={K}")
    if S.shape != (K // G, N):
        raise ValueError(f"scales shape {S.shape} != {(K // G, N)}")
    if QZ is not None and (N % 8 != 0 or QZ.shape != (K // G, N // 8)):
        raise ValueError(f"qzeros shape {QZ.shape} does not pack N={N} columns in groups of 8")


class Oracle:
    """numpy-facing wrapper of one compiled oracle library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_h2d.restype = ctypes.c_double
        lib.oracle_h2d.argtypes = [ctypes.c_uint16]
        lib.oracle_d2h.restype = ctypes.c_uint16
        lib.oracle_d2h.argtypes = [ctypes.c_double]
        lib.oracle_h2d_n.argtypes = [_u16p, ctypes.c_size_t, _f64p]
        lib.oracle_d2h_n.argtypes = [_f64p, ctypes.c_size_t, _u16p]
        lib.oracle_pack.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, _i32p]
        lib.oracle_pack_zeros.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, _i32p]
        lib.oracle_unpack.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, _u8p]
        lib.oracle_unpack_zeros.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, _u8p]
        lib.oracle_interleave.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, _i32p]
        lib.oracle_deinterleave.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, _i32p]
        lib.oracle_block.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, _i32p]
        lib.oracle_unblock.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, _i32p]
        lib.oracle_dequant_one.restype = ctypes.c_uint16
        lib.oracle_dequant_one.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint16]
        lib.oracle_dequant.argtypes = [_i32p, _u16p, _i32p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, _u16p]
        lib.oracle_matmul_w.argtypes = [_u16p, _u16p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, _f64p, _u16p]
        lib.oracle_quantize.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, _u8p, _u16p, _u8p]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_gate_up.argtypes = [_f64p, ctypes.c_int, ctypes.c_int, _u16p]
        I, D = ctypes.c_int, ctypes.c_double
        lib.oracle_channel_stats.argtypes = [_u16p, I, _u16p, I, I, I, _f64p, _f64p]
        lib.oracle_scale_candidate.argtypes = [_f64p, _f64p, I, D, _f64p]
        lib.oracle_migrate.argtypes = [_u16p, _u16p, I, I, I, _f64p, _u16p, _u16p]
        lib.oracle_scale_loss.restype = I
        lib.oracle_scale_loss.argtypes = [_u16p, _u16p, I, I, I, I, I, _f64p,
                                          ctypes.POINTER(ctypes.c_double)]
        lib.oracle_scale_search.restype = I
        lib.oracle_scale_search.argtypes = [_u16p, I, _u16p, I, I, I, I, _f64p, I, _f64p, _f64p]
        lib.oracle_linear.restype = ctypes.c_int
        lib.oracle_linear.argtypes = [_u16p, _i32p, _u16p, _i32p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, _f64p, _u16p]
        self.lib = lib

    # -- fp16 codec ---------------------------------------------------------
    def h2d(self, h: int) -> float:
        return self.lib.oracle_h2d(int(h) & 0xFFFF)

    def d2h(self, x: float) -> int:
        return int(self.lib.oracle_d2h(float(x)))

    def h2d_array(self, h: np.ndarray) -> np.ndarray:
        flat = np.ascontiguousarray(h, dtype=np.uint16).ravel()
        out = np.empty(flat.size, dtype=np.float64)
        self.lib.oracle_h2d_n(_ptr(flat, _u16p), flat.size, _ptr(out, _f64p))
        return out.reshape(np.shape(h))

    def d2h_array(self, x: np.ndarray) -> np.ndarray:
        flat = np.ascontiguousarray(x, dtype=np.float64).ravel()
        out = np.empty(flat.size, dtype=np.uint16)
        self.lib.oracle_d2h_n(_ptr(flat, _f64p), flat.size, _ptr(out, _u16p))
        return out.reshape(np.shape(x))

    # -- packing --------------------------------------------------------------
    def pack(self, codes: np.ndarray) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        K, N = codes.shape
        if K % 8 != 0:
            raise ValueError(f"K={K} is not a multiple of 8 codes per word")
        Q = np.empty((K // 8, N), dtype=np.int32)
        self.lib.oracle_pack(_ptr(codes, _u8p), K, N, _ptr(Q, _i32p))
        return Q

    def pack_zeros(self, zeros: np.ndarray) -> np.ndarray:
        zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
        groups, N = zeros.shape
        if N % 8 != 0:
            raise ValueError(f"N={N} is not a multiple of 8 zero points per word")
        QZ = np.empty((groups, N // 8), dtype=np.int32)
        self.lib.oracle_pack_zeros(_ptr(zeros, _u8p), groups, N, _ptr(QZ, _i32p))
        return QZ

    def unpack(self, Q: np.ndarray) -> np.ndarray:
        Q = np.ascontiguousarray(Q, dtype=np.int32)
        R, N = Q.shape
        codes = np.empty((8 * R, N), dtype=np.uint8)
        self.lib.oracle_unpack(_ptr(Q, _i32p), 8 * R, N, _ptr(codes, _u8p))
        return codes

    def unpack_zeros(self, QZ: np.ndarray) -> np.ndarray:
        QZ = np.ascontiguousarray(QZ, dtype=np.int32)
        groups, C = QZ.shape
        zeros = np.empty((groups, 8 * C), dtype=np.uint8)
        self.lib.oracle_unpack_zeros(_ptr(QZ, _i32p), groups, 8 * C, _ptr(zeros, _u8p))
        return zeros

    # -- kernel-private layout (R17) ------------------------------------------
    def interleave(self, Q: np.ndarray) -> np.ndarray:
        """Canonical packed words -> the interleaved layout (even k in the low
        half-word, odd k in the high half-word)."""
        Q = np.ascontiguousarray(Q, dtype=np.int32)
        out = np.empty_like(Q)
        self.lib.oracle_interleave(_ptr(Q, _i32p), 8 * Q.shape[0], Q.shape[1], _ptr(out, _i32p))
        return out

    def deinterleave(self, Q: np.ndarray) -> np.ndarray:
        """The inverse of ``interleave``."""
        Q = np.ascontiguousarray(Q, dtype=np.int32)
        out = np.empty_like(Q)
        self.lib.oracle_deinterleave(_ptr(Q, _i32p), 8 * Q.shape[0], Q.shape[1], _ptr(out, _i32p))
        return out

    def block(self, Q: np.ndarray) -> np.ndarray:
        """Packed words [K/8][N] -> their places in 128-column blocks (R18), as a
        flat int32 array of K/8 * N words; nibbles untouched."""
        Q = np.ascontiguousarray(Q, dtype=np.int32)
        if Q.shape[1] % 128:
            raise ValueError("the blocked layout needs N % 128 == 0")
        out = np.empty(Q.size, dtype=np.int32)
        self.lib.oracle_block(_ptr(Q, _i32p), 8 * Q.shape[0], Q.shape[1], _ptr(out, _i32p))
        return out

    def unblock(self, B: np.ndarray, K: int, N: int) -> np.ndarray:
        """The inverse of ``block``: [K/8][N] words from a flat blocked array."""
        B = np.ascontiguousarray(B, dtype=np.int32).reshape(-1)
        if N % 128 or B.size != (K // 8) * N:
            raise ValueError("the blocked layout needs N % 128 == 0 and K/8 * N words")
        out = np.empty((K // 8, N), dtype=np.int32)
        self.lib.oracle_unblock(_ptr(B, _i32p), K, N, _ptr(out, _i32p))
        return out

    # -- dequantization -------------------------------------------------------
    def dequant_one(self, q: int, z: int, s: int) -> int:
        return int(self.lib.oracle_dequant_one(int(q), int(z), int(s) & 0xFFFF))

    def dequant(self, Q: np.ndarray, S: np.ndarray, QZ: np.ndarray | None, G: int) -> np.ndarray:
        Q = np.ascontiguousarray(Q, dtype=np.int32)
        S = np.ascontiguousarray(S, dtype=np.uint16)
        if QZ is not None:
            QZ = np.ascontiguousarray(QZ, dtype=np.int32)
        K, N = 8 * Q.shape[0], Q.shape[1]
        _check_layer(K, N, G, S, QZ)
        W = np.empty((K, N), dtype=np.uint16)
        self.lib.oracle_dequant(_ptr(Q, _i32p), _ptr(S, _u16p), _ptr(QZ, _i32p), K, N, G,
                                _ptr(W, _u16p))
        return W

    # -- the layer ------------------------------------------------------------
    def matmul_w(self, X: np.ndarray, W: np.ndarray):
        X = np.ascontiguousarray(X, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.uint16)
        M, K = X.shape
        N = W.shape[1]
        Y64 = np.empty((M, N), dtype=np.float64)
        Y16 = np.empty((M, N), dtype=np.uint16)
        self.lib.oracle_matmul_w(_ptr(X, _u16p), _ptr(W, _u16p), M, K, N, _ptr(Y64, _f64p),
                                 _ptr(Y16, _u16p))
        return Y64, Y16

    def linear(self, X: np.ndarray, Q: np.ndarray, S: np.ndarray, QZ: np.ndarray | None,
               G: int):
        """Y = X @ dequant(Q, S, QZ); returns (Y64 fp64, Y16 fp16 bit patterns)."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        Q = np.ascontiguousarray(Q, dtype=np.int32)
        S = np.ascontiguousarray(S, dtype=np.uint16)
        if QZ is not None:
            QZ = np.ascontiguousarray(QZ, dtype=np.int32)
        M, K = X.shape
        N = Q.shape[1]
        if Q.shape[0] * 8 != K:
            raise ValueError(f"qweight has {Q.shape[0]} packed rows for K={K}")
        _check_layer(K, N, G, S, QZ)
        Y64 = np.empty((M, N), dtype=np.float64)
        Y16 = np.empty((M, N), dtype=np.uint16)
        rc = self.lib.oracle_linear(_ptr(X, _u16p), _ptr(Q, _i32p), _ptr(S, _u16p),
                                    _ptr(QZ, _i32p), M, K, N, G, _ptr(Y64, _f64p),
                                    _ptr(Y16, _u16p))
        if rc != 0:
            raise MemoryError("oracle_linear could not allocate the dequantized weight")
        return Y64, Y16


    def linear_columns(self, X: np.ndarray, Q: np.ndarray, S: np.ndarray,
                       QZ: np.ndarray | None, G: int, threads: int):
        """``linear`` computed over column slices by ``threads`` host threads.

        Each output column is summed by one call over its own slice of the layer,
        in the same increasing-k order, so the result is bit-identical to
        ``linear``; only the columns are spread over threads (the C calls run
        without the GIL)."""
        Q = np.ascontiguousarray(Q, dtype=np.int32)
        S = np.ascontiguousarray(S, dtype=np.uint16)
        M, N = X.shape[0], Q.shape[1]
        if threads <= 1 or N < 16:
            return self.linear(X, Q, S, QZ, G)
        blocks = N // 8
        cuts = [8 * (blocks * i // threads) for i in range(threads + 1)]
        Y64 = np.empty((M, N), dtype=np.float64)
        Y16 = np.empty((M, N), dtype=np.uint16)

        def part(i):
            a, b = cuts[i], cuts[i + 1]
            if a == b:
                return
            qz = None if QZ is None else QZ[:, a // 8:b // 8]
            y64, y16 = self.linear(X, Q[:, a:b], S[:, a:b], qz, G)
            Y64[:, a:b], Y16[:, a:b] = y64, y16

        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(part, range(threads)))
        return Y64, Y16

    def matmul_w_columns(self, X: np.ndarray, W: np.ndarray, threads: int):
        """``matmul_w`` over column slices of W on ``threads`` host threads
        (bit-identical: every column keeps its increasing-k sum)."""
        M, N = X.shape[0], W.shape[1]
        if threads <= 1 or N < 16:
            return self.matmul_w(X, W)
        cuts = [N * i // threads for i in range(threads + 1)]
        Y64 = np.empty((M, N), dtype=np.float64)
        Y16 = np.empty((M, N), dtype=np.uint16)

        def part(i):
            a, b = cuts[i], cuts[i + 1]
            if a < b:
                Y64[:, a:b], Y16[:, a:b] = self.matmul_w(X, W[:, a:b])

        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(part, range(threads)))
        return Y64, Y16

    # -- quantizer ------------------------------------------------------------
    def quantize(self, W: np.ndarray, G: int, symmetric: bool):
        """fp16 W[K][N] -> (codes u8 [K][N], scales fp16 [K/G][N], zeros u8 [K/G][N] or None)."""
        W = np.ascontiguousarray(W, dtype=np.uint16)
        K, N = W.shape
        if G <= 0 or K % G != 0:
            raise ValueError(f"group size {G} must divide K={K}")
        codes = np.empty((K, N), dtype=np.uint8)
        S = np.empty((K // G, N), dtype=np.uint16)
        Z = None if symmetric else np.empty((K // G, N), dtype=np.uint8)
        self.lib.oracle_quantize(_ptr(W, _u16p), K, N, G, int(symmetric), _ptr(codes, _u8p),
                                 _ptr(S, _u16p), _ptr(Z, _u8p))
        return codes, S, Z

    # -- fused gate/up epilogue ---------------------------------------------
    def silu(self, t: float) -> float:
        return self.lib.oracle_silu(float(t))

    def gate_up(self, Y64: np.ndarray) -> np.ndarray:
        """h = fp16(SiLU(Y64[:, :I]) * Y64[:, I:]) from the layer's fp64 sums."""
        Y64 = np.ascontiguousarray(Y64, dtype=np.float64)
        M, N = Y64.shape
        if N % 2 != 0:
            raise ValueError(f"N={N} is not [gate | up] with equal halves")
        H16 = np.empty((M, N // 2), dtype=np.uint16)
        self.lib.oracle_gate_up(_ptr(Y64, _f64p), M, N // 2, _ptr(H16, _u16p))
        return H16

    # -- scale migration and search (R14, R15, R16) ---------------------------
    def channel_stats(self, X: np.ndarray, W: np.ndarray, G: int):
        """(xbar, wbar) fp64 [K]: mean |x| per input channel, and the mean over
        output columns of |w| normalized by its group's largest |w|."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.uint16)
        M, K = X.shape
        N = W.shape[1]
        if W.shape[0] != K or G <= 0 or K % G != 0:
            raise ValueError(f"X {X.shape}, W {W.shape}, G={G} do not fit")
        xbar, wbar = np.empty(K), np.empty(K)
        self.lib.oracle_channel_stats(_ptr(X, _u16p), M, _ptr(W, _u16p), K, N, G,
                                      _ptr(xbar, _f64p), _ptr(wbar, _f64p))
        return xbar, wbar

    def scale_candidate(self, xbar: np.ndarray, wbar: np.ndarray, alpha: float) -> np.ndarray:
        xbar = np.ascontiguousarray(xbar, dtype=np.float64)
        wbar = np.ascontiguousarray(wbar, dtype=np.float64)
        c = np.empty(xbar.size)
        self.lib.oracle_scale_candidate(_ptr(xbar, _f64p), _ptr(wbar, _f64p), xbar.size,
                                        float(alpha), _ptr(c, _f64p))
        return c

    def migrate(self, X: np.ndarray, W: np.ndarray, c: np.ndarray):
        """(fp16(X / c), fp16(c * W)), c per input channel."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.uint16)
        c = np.ascontiguousarray(c, dtype=np.float64)
        M, K = X.shape
        N = W.shape[1]
        if W.shape[0] != K or c.size != K:
            raise ValueError("X, W and c do not fit")
        Xs, Ws = np.empty_like(X), np.empty_like(W)
        self.lib.oracle_migrate(_ptr(X, _u16p), _ptr(W, _u16p), M, K, N, _ptr(c, _f64p),
                                _ptr(Xs, _u16p), _ptr(Ws, _u16p))
        return Xs, Ws

    def scale_loss(self, X: np.ndarray, W: np.ndarray, G: int, symmetric: bool,
                   c: np.ndarray) -> float:
        X = np.ascontiguousarray(X, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.uint16)
        c = np.ascontiguousarray(c, dtype=np.float64)
        M, K = X.shape
        N = W.shape[1]
        if W.shape[0] != K or c.size != K or G <= 0 or K % G != 0:
            raise ValueError("X, W, c and G do not fit")
        out = ctypes.c_double()
        if self.lib.oracle_scale_loss(_ptr(X, _u16p), _ptr(W, _u16p), M, K, N, G,
                                      int(symmetric), _ptr(c, _f64p), ctypes.byref(out)) != 0:
            raise MemoryError("oracle_scale_loss could not allocate")
        return out.value

    def scale_search(self, X: np.ndarray, W: np.ndarray, G: int, symmetric: bool, alphas):
        """(best index, losses fp64 [n_alpha], scales of the best alpha fp64 [K])."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.uint16)
        a = np.ascontiguousarray(alphas, dtype=np.float64)
        M, K = X.shape
        N = W.shape[1]
        if W.shape[0] != K or G <= 0 or K % G != 0 or a.size < 1:
            raise ValueError("X, W, G and alphas do not fit")
        losses, c = np.empty(a.size), np.empty(K)
        best = self.lib.oracle_scale_search(_ptr(X, _u16p), M, _ptr(W, _u16p), K, N, G,
                                            int(symmetric), _ptr(a, _f64p), a.size,
                                            _ptr(losses, _f64p), _ptr(c, _f64p))
        if best < 0:
            raise MemoryError("oracle_scale_search could not allocate")
        return best, losses, c


_DEFAULT: Oracle | None = None


def load() -> Oracle:
    """The oracle built from ``oracle.c`` beside this file (built on first use)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT
