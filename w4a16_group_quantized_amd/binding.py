"""Thin Python binding over libawq.so (C ABI of include/awq.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream; tensors must
be contiguous, on the GPU, and of the dtypes below.  If the library has not
been built, the first call raises -- there is no fallback path.

Layout (see include/awq.h): qweight int32 [K/8][N], scales fp16 [K/G][N],
qzeros int32 [K/G][N/8] or None (symmetric), x fp16 [M][K], y fp16 [M][N].
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libawq.so")

# Entry points declared in include/awq.h, in declaration order.
ENTRY_POINTS = ("awq_status_string", "awq_pack", "awq_pack_zeros", "awq_repack", "awq_dequant",
                "awq_gemv_workspace_bytes", "awq_gemv",
                "awq_gemm", "awq_gemv_gate_up", "awq_quantize", "awq_gemm_gate_up",
                "awq_gemm_splitk_workspace_bytes", "awq_gemm_splitk", "awq_gemm_splitk_static",
                "awq_channel_stats_workspace_bytes", "awq_channel_stats",
                "awq_scale_search_workspace_bytes", "awq_scale_search")

# awq_status values of include/awq.h
AWQ_SUCCESS = 0
AWQ_ERROR_INVALID_VALUE = 1
AWQ_ERROR_SHAPE = 2
AWQ_ERROR_ALIGNMENT = 3
AWQ_ERROR_UNSUPPORTED = 4
AWQ_ERROR_WORKSPACE = 5
AWQ_ERROR_HIP = 6
STATUS_NAMES = {AWQ_SUCCESS: "AWQ_SUCCESS", AWQ_ERROR_INVALID_VALUE: "AWQ_ERROR_INVALID_VALUE",
                AWQ_ERROR_SHAPE: "AWQ_ERROR_SHAPE", AWQ_ERROR_ALIGNMENT: "AWQ_ERROR_ALIGNMENT",
                AWQ_ERROR_UNSUPPORTED: "AWQ_ERROR_UNSUPPORTED",
                AWQ_ERROR_WORKSPACE: "AWQ_ERROR_WORKSPACE", AWQ_ERROR_HIP: "AWQ_ERROR_HIP"}
SCALE_SEARCH_MAX_ALPHAS = 64
# qweight layouts (AWQ_LAYOUT_* of include/awq.h)
LAYOUT_CANONICAL = 0
LAYOUT_INTERLEAVED = 1
LAYOUT_BLOCKED = 2        # interleaved words, 128-column blocks contiguous (N % 128 == 0)


class AwqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class CLayer(ctypes.Structure):
    """``awq_layer`` of include/awq.h."""

    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("qzeros", ctypes.c_void_p), ("K", ctypes.c_int32), ("N", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("layout", ctypes.c_int32)]


_LIB = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libawq.so and declare its signatures (raises if it is missing)."""
    global _LIB
    if _LIB is not None and path == LIBRARY:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m w4a16_group_quantized_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.awq_status_string.restype = ctypes.c_char_p
    lib.awq_status_string.argtypes = [ctypes.c_int]
    lib.awq_pack.restype = ctypes.c_int
    lib.awq_pack.argtypes = [vp, vp, i32, i32, vp]
    lib.awq_pack_zeros.restype = ctypes.c_int
    lib.awq_pack_zeros.argtypes = [vp, vp, i32, i32, vp]
    lib.awq_repack.restype = ctypes.c_int
    lib.awq_repack.argtypes = [vp, vp, i32, i32, i32, i32, vp]
    lib.awq_dequant.restype = ctypes.c_int
    lib.awq_dequant.argtypes = [ctypes.POINTER(CLayer), vp, vp]
    lib.awq_quantize.restype = ctypes.c_int
    lib.awq_quantize.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp]
    for name in ("awq_gemm", "awq_gemv_gate_up", "awq_gemm_gate_up"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, ctypes.POINTER(CLayer), vp, i32, vp]
    lib.awq_gemv_workspace_bytes.restype = ctypes.c_size_t
    lib.awq_gemv_workspace_bytes.argtypes = [i32, i32, i32]
    lib.awq_gemv.restype = ctypes.c_int
    lib.awq_gemv.argtypes = [vp, ctypes.POINTER(CLayer), vp, i32, vp, ctypes.c_size_t, vp]
    lib.awq_gemm_splitk_workspace_bytes.restype = ctypes.c_size_t
    lib.awq_gemm_splitk_workspace_bytes.argtypes = [i32, i32, i32]
    lib.awq_gemm_splitk.restype = ctypes.c_int
    lib.awq_gemm_splitk.argtypes = [vp, ctypes.POINTER(CLayer), vp, i32, i32, vp, ctypes.c_size_t, vp]
    lib.awq_gemm_splitk_static.restype = ctypes.c_int
    lib.awq_gemm_splitk_static.argtypes = [vp, ctypes.POINTER(CLayer), vp, i32, i32, vp]
    for name in ("awq_channel_stats_workspace_bytes", "awq_scale_search_workspace_bytes"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_size_t
        fn.argtypes = [i32, i32, i32, i32]
    lib.awq_channel_stats.restype = ctypes.c_int
    lib.awq_channel_stats.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.awq_scale_search.restype = ctypes.c_int
    lib.awq_scale_search.argtypes = [vp, i32, vp, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_float),
                                     i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    if path == LIBRARY:
        _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().awq_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != AWQ_SUCCESS:
        raise AwqError(status, status_string(status))


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _new(shape, dtype: torch.dtype, device, stream=None) -> torch.Tensor:
    """torch.empty for an output or workspace of a call enqueued on ``stream``.
    The caching allocator ties a block to the stream current at allocation; when
    the kernels run on another stream, the block is recorded on that stream too,
    so it is not handed out again before they are done."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


@dataclass
class Layer:
    """One quantized linear layer resident on the GPU (logical weight W[K][N])."""

    qweight: torch.Tensor            # int32 [K/8][N]
    scales: torch.Tensor             # fp16  [K/G][N]
    qzeros: torch.Tensor | None      # int32 [K/G][N/8] or None (symmetric)
    K: int
    N: int
    group_size: int
    layout: int = LAYOUT_CANONICAL   # of qweight (LAYOUT_*)

    def c_struct(self) -> CLayer:
        """The C view, after checking that the tensors have the shapes K, N and
        group_size imply and sit on one device (the library trusts both)."""
        K, N, G = self.K, self.N, self.group_size
        if G > 0 and K > 0 and K % G == 0 and K % 8 == 0 and N % 8 == 0:
            want = {"qweight": (K // 8, N), "scales": (K // G, N), "qzeros": (K // G, N // 8)}
            for name, t in (("qweight", self.qweight), ("scales", self.scales),
                            ("qzeros", self.qzeros)):
                if t is not None and tuple(t.shape) != want[name]:
                    raise ValueError(f"{name} must be {list(want[name])} for K={K} N={N} "
                                     f"G={G}, got {list(t.shape)}")
        for name, t in (("scales", self.scales), ("qzeros", self.qzeros)):
            if t is not None and t.device != self.qweight.device:
                raise ValueError(f"{name} is on {t.device}, qweight on {self.qweight.device}")
        qw = _dev(self.qweight, torch.int32, "qweight")
        sc = _dev(self.scales, torch.float16, "scales")
        qz = None if self.qzeros is None else _dev(self.qzeros, torch.int32, "qzeros")
        return CLayer(qw, sc, qz, K, N, G, self.layout)

    @property
    def device(self) -> torch.device:
        return self.qweight.device


def pack(codes: torch.Tensor, stream=None) -> torch.Tensor:
    """uint8 codes [K][N] -> int32 qweight [K/8][N]."""
    K, N = codes.shape
    out = _new((K // 8, N), torch.int32, codes.device, stream)
    _check(load().awq_pack(_dev(codes, torch.uint8, "codes"), out.data_ptr(), K, N,
                           _stream(stream)))
    return out


def pack_zeros(zeros: torch.Tensor, stream=None) -> torch.Tensor:
    """uint8 zeros [K/G][N] -> int32 qzeros [K/G][N/8]."""
    groups, N = zeros.shape
    out = _new((groups, N // 8), torch.int32, zeros.device, stream)
    _check(load().awq_pack_zeros(_dev(zeros, torch.uint8, "zeros"), out.data_ptr(), groups, N,
                                 _stream(stream)))
    return out


def repack_words(qweight: torch.Tensor, to: int, frm: int = LAYOUT_CANONICAL,
                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Packed words int32 [K/8][N] from layout ``frm`` to layout ``to`` (LAYOUT_*);
    ``out`` may be ``qweight`` itself (in place) unless exactly one of the two
    layouts is LAYOUT_BLOCKED, which moves words."""
    R, N = qweight.shape
    if out is None:
        out = _new((R, N), torch.int32, qweight.device, stream)
    elif tuple(out.shape) != (R, N):
        raise ValueError(f"out must be [{R}][{N}], got {tuple(out.shape)}")
    _check(load().awq_repack(_dev(qweight, torch.int32, "qweight"), _dev(out, torch.int32, "out"),
                             8 * R, N, frm, to, _stream(stream)))
    return out


def repack(layer: Layer, to: int = LAYOUT_INTERLEAVED, stream=None) -> Layer:
    """The same layer with its packed words in layout ``to`` (a new qweight)."""
    q = repack_words(layer.qweight, to, layer.layout, stream=stream)
    return Layer(q, layer.scales, layer.qzeros, layer.K, layer.N, layer.group_size, to)


def make_layer(codes: torch.Tensor, zeros: torch.Tensor | None, scales: torch.Tensor,
               group_size: int, stream=None) -> Layer:
    """Packs device codes/zeros (uint8) into a Layer; scales are fp16 [K/G][N]."""
    K, N = codes.shape
    qz = None if zeros is None else pack_zeros(zeros, stream)
    return Layer(pack(codes, stream), scales, qz, K, N, group_size)


def gemm_gate_up(x: torch.Tensor, layer: Layer, out: torch.Tensor | None = None, stream=None):
    """h = SiLU(y[:, :N/2]) * y[:, N/2:] with y = x @ dequant(layer), any M; the layer's
    columns are the concatenation [gate | up]."""
    return _linear("awq_gemm_gate_up", x, layer, out, stream, width=layer.N // 2)


def quantize(w: torch.Tensor, group_size: int, symmetric: bool = False, stream=None) -> Layer:
    """fp16 W[K][N] -> a Layer (packed codes, scales, zero points or None), by
    per-group min-max."""
    K, N = w.shape
    dev = w.device
    qweight = _new((K // 8, N), torch.int32, dev, stream)
    scales = _new((K // group_size, N), torch.float16, dev, stream)
    qzeros = None if symmetric else _new((K // group_size, N // 8), torch.int32, dev, stream)
    _check(load().awq_quantize(_dev(w, torch.float16, "w"), K, N, group_size, int(symmetric),
                               qweight.data_ptr(), scales.data_ptr(),
                               None if qzeros is None else qzeros.data_ptr(), _stream(stream)))
    return Layer(qweight, scales, qzeros, K, N, group_size)


def dequant(layer: Layer, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Exact fp16 W[K][N]."""
    c = layer.c_struct()
    if out is None:
        out = _new((layer.K, layer.N), torch.float16, layer.device, stream)
    _check(load().awq_dequant(ctypes.byref(c), _dev(out, torch.float16, "out"), _stream(stream)))
    return out


def _io(x: torch.Tensor, layer: Layer, out: torch.Tensor | None, stream, width: int):
    """Checks x [M][K] (and out [M][width]) against the layer; allocates out."""
    if x.dim() != 2 or x.shape[1] != layer.K:
        raise ValueError(f"x must be [M][{layer.K}], got {tuple(x.shape)}")
    c = layer.c_struct()
    if x.device != layer.device:
        raise ValueError(f"x is on {x.device}, the layer on {layer.device}")
    M = x.shape[0]
    if out is None:
        out = _new((M, width), torch.float16, x.device, stream)
    elif tuple(out.shape) != (M, width) or out.device != x.device:
        raise ValueError(f"out must be [{M}][{width}] on {x.device}, got {tuple(out.shape)} "
                         f"on {out.device}")
    return M, c, out


def _linear(fn_name: str, x: torch.Tensor, layer: Layer, out: torch.Tensor | None, stream,
            width: int | None = None):
    M, c, out = _io(x, layer, out, stream, layer.N if width is None else width)
    _check(getattr(load(), fn_name)(_dev(x, torch.float16, "x"), ctypes.byref(c),
                                    _dev(out, torch.float16, "out"), M, _stream(stream)))
    return out


def gemv(x: torch.Tensor, layer: Layer, out: torch.Tensor | None = None, stream=None,
         workspace: torch.Tensor | None = None):
    """y = x @ dequant(layer) for 1 <= M <= 16 (decode).  The library asks for no
    workspace here (awq_gemv_workspace_bytes is 0); one may still be passed."""
    M, c, out = _io(x, layer, out, stream, layer.N)
    lib = load()
    need = lib.awq_gemv_workspace_bytes(M, layer.K, layer.N)
    if workspace is None and need > 0:
        workspace = _new(need, torch.uint8, x.device, stream)
    ws = None if workspace is None else _dev(workspace, torch.uint8, "workspace")
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib.awq_gemv(_dev(x, torch.float16, "x"), ctypes.byref(c),
                        _dev(out, torch.float16, "out"), M, ws, nbytes, _stream(stream)))
    return out


def gemm(x: torch.Tensor, layer: Layer, out: torch.Tensor | None = None, stream=None):
    """y = x @ dequant(layer) for any M (prefill / batches)."""
    return _linear("awq_gemm", x, layer, out, stream)


def splitk_splits(M: int, layer: Layer, cus: int = 256) -> int:
    """Slices of K for awq_gemm_splitk (1, 2, 4, 8 or 16, among those the layer
    allows).

    Up to 64 rows the kernel takes 64-row tiles, and the rule is measured: the
    most slices that keep at least 512 k per slice and at most 448 workgroups
    (256 beyond 32 rows).  Over 14 MI355X shapes (K 4096 to 14336, N 4096 to
    28672, M 16 to 64) it lands within 9% of the best count, 1.5% on average.

    Beyond 64 rows, a cost model fitted to MI355X timings of a 4096 x 4096 and a
    4096 x 28672 layer at M = 128 to 2048.  Workgroups (128 x 256 output tiles
    times slices) run in waves of one per CU; a workgroup costs about 3.2 us
    plus 8.8 ns per k, the per-k cost growing by up to 57% as the wave fills the
    chip (the MFMA units share the power budget); a split adds about 5.9 us and
    the partial sums, splits * M * N * 4 bytes written and read again at about
    7.9 TB/s.  More slices are taken only where the model saves at least 5%."""
    def allowed(s):
        # the library's rule (AWQ_ERROR_UNSUPPORTED otherwise): slices of
        # whole groups (or inside the single group), in whole ring turns of
        # 64-k steps (G a multiple of 64) or of 32-k steps (G of 32)
        if layer.K % s:
            return False
        ks, G = layer.K // s, layer.group_size
        one = G == layer.K
        whole = one or ks % G == 0
        return whole and (((one or G % 64 == 0) and ks % 256 == 0) or
                          ((one or G % 32 == 0) and ks % 128 == 0))

    if M <= 64:
        tiles = -(-layer.N // 256)
        cap = 448 if M <= 32 else 256
        best = 1
        for s in (2, 4, 8, 16):
            if allowed(s) and tiles * s <= cap and layer.K // s >= 512:
                best = s
        return best

    tiles = -(-M // 128) * -(-layer.N // 256)

    def cost(s):
        active = min(tiles * s, cus)
        waves = -(-tiles * s // cus)
        t = waves * (3.2e-6 + (layer.K // s) * 8.8e-9 * (1 + 0.57 * active / cus))
        if s > 1:
            t += 5.9e-6 + 2 * s * M * layer.N * 4 / 7.9e12
        return t

    best = 1
    for s in (2, 4, 8, 16):
        if allowed(s) and cost(s) < 0.95 * cost(best):
            best = s
    return best


def gemm_splitk(x: torch.Tensor, layer: Layer, splits: int | None = None,
                out: torch.Tensor | None = None, stream=None, workspace: torch.Tensor | None = None):
    """awq_gemm's output with K split across workgroups (``splits`` slices, chosen by
    splitk_splits when None); the fp32 partials go to ``workspace`` (allocated here
    unless given)."""
    M, c, out = _io(x, layer, out, stream, layer.N)
    splits = splitk_splits(M, layer) if splits is None else splits
    lib = load()
    if workspace is None:
        nbytes = lib.awq_gemm_splitk_workspace_bytes(max(M, 1), layer.N, splits)
        workspace = _new(max(nbytes, 16), torch.uint8, x.device, stream)
    _check(lib.awq_gemm_splitk(_dev(x, torch.float16, "x"), ctypes.byref(c),
                               _dev(out, torch.float16, "out"), M, splits,
                               _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                               _stream(stream)))
    return out


# Size of the library's static split-K scratch (AWQ_GEMM_SPLITK_STATIC_SCRATCH_BYTES).
GEMM_SPLITK_STATIC_SCRATCH_BYTES = 32 << 20


def gemm_splitk_static(x: torch.Tensor, layer: Layer, splits: int, out: torch.Tensor,
                       stream=None):
    """awq_gemm_splitk's output on the library's static per-device scratch: the
    call allocates nothing (``out`` is required).  Calls overlapping in time on
    one GPU share that scratch and race."""
    if out is None:
        raise ValueError("gemm_splitk_static allocates nothing: pass out [M][N]")
    M, c, out = _io(x, layer, out, stream, layer.N)
    _check(load().awq_gemm_splitk_static(_dev(x, torch.float16, "x"), ctypes.byref(c),
                                         _dev(out, torch.float16, "out"), M, splits,
                                         _stream(stream)))
    return out


def gemv_gate_up(x: torch.Tensor, layer: Layer, out: torch.Tensor | None = None, stream=None):
    """h = SiLU(y[:, :N/2]) * y[:, N/2:] with y = x @ dequant(layer), 1 <= M <= 16; the
    layer's columns are the concatenation [gate | up]."""
    return _linear("awq_gemv_gate_up", x, layer, out, stream, width=layer.N // 2)


def _calibration(x: torch.Tensor, w: torch.Tensor):
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[0]:
        raise ValueError(f"x [M][K] and w [K][N] do not fit: {tuple(x.shape)}, {tuple(w.shape)}")
    return x.shape[0], w.shape[0], w.shape[1]


def channel_stats(x: torch.Tensor, w: torch.Tensor, group_size: int, stream=None):
    """(xbar, wbar) fp32 [K]: mean |x| per input channel over the calibration rows,
    and the mean over output columns of |w| over its group's largest |w|."""
    M, K, N = _calibration(x, w)
    lib = load()
    xbar = _new(K, torch.float32, x.device, stream)
    wbar = _new(K, torch.float32, x.device, stream)
    nbytes = lib.awq_channel_stats_workspace_bytes(M, K, N, group_size)
    ws = _new(max(nbytes, 16), torch.uint8, x.device, stream)
    _check(lib.awq_channel_stats(_dev(x, torch.float16, "x"), M, _dev(w, torch.float16, "w"), K, N,
                                 group_size, xbar.data_ptr(), wbar.data_ptr(), ws.data_ptr(),
                                 ws.numel(), _stream(stream)))
    return xbar, wbar


def scale_search(x: torch.Tensor, w: torch.Tensor, group_size: int, alphas, symmetric: bool = False,
                 stream=None, workspace: torch.Tensor | None = None):
    """AWQ's scale search over the grid ``alphas``: (best index as a device int32
    tensor, losses fp64 [n_alpha], scales fp32 [K] of the best alpha).  The
    workspace is allocated here unless one of at least
    awq_scale_search_workspace_bytes is given."""
    M, K, N = _calibration(x, w)
    lib = load()
    a = (ctypes.c_float * len(alphas))(*[float(v) for v in alphas])
    losses = _new(len(alphas), torch.float64, x.device, stream)
    best = _new(1, torch.int32, x.device, stream)
    scales = _new(K, torch.float32, x.device, stream)
    if workspace is None:
        nbytes = lib.awq_scale_search_workspace_bytes(M, K, N, group_size)
        workspace = _new(max(nbytes, 16), torch.uint8, x.device, stream)
    _check(lib.awq_scale_search(_dev(x, torch.float16, "x"), M, _dev(w, torch.float16, "w"), K, N,
                                group_size, int(symmetric), a, len(alphas), losses.data_ptr(),
                                best.data_ptr(), scales.data_ptr(),
                                _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                _stream(stream)))
    return best, losses, scales

