"""The C-ABI library on the CPU: it loads, exports every entry point that
include/awq.h declares, and rejects bad arguments before touching a GPU.

Only invalid argument combinations are passed (or M == 0, which returns before
any launch), so nothing here launches a kernel; the fake device addresses are
never dereferenced.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from w4a16_group_quantized_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")

FAKE = 0x10000000          # 16-byte aligned, never dereferenced
MISALIGNED = FAKE + 2
WS = binding.AWQ_ERROR_WORKSPACE


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_header_matches_binding():
    assert header_functions() == sorted(binding.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (awq_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code, name in binding.STATUS_NAMES.items():
        assert lib.awq_status_string(code).decode().startswith(name)
    assert lib.awq_status_string(99).decode() == "AWQ_ERROR_UNKNOWN"


def layer(K=128, N=64, G=128, qw=FAKE, sc=FAKE, qz=FAKE, layout=0):
    return binding.CLayer(qw, sc, qz, K, N, G, layout)


def _call(lib, fn, x, c, y, M):
    """One layer call; awq_gemv also takes its (empty) workspace."""
    if fn == "awq_gemv":
        return lib.awq_gemv(x, c, y, M, None, 0, None)
    return getattr(lib, fn)(x, c, y, M, None)


@pytest.mark.parametrize("fn", ["awq_gemv", "awq_gemm", "awq_gemv_gate_up", "awq_gemm_gate_up"])
@pytest.mark.parametrize("case,want", [
    (dict(K=0), 1), (dict(N=-8), 1), (dict(G=0), 1),
    (dict(K=12), 2), (dict(N=20), 2), (dict(G=12, K=24), 2), (dict(K=192, G=128), 2),
    (dict(K=1 << 16, N=1 << 16, G=128), 2),
    (dict(qw=None), 1), (dict(sc=None), 1),
    (dict(qw=MISALIGNED), 3), (dict(sc=MISALIGNED), 3), (dict(qz=MISALIGNED), 3),
    (dict(layout=3), 1), (dict(layout=-1), 1),
    (dict(layout=2), 2),                       # blocked words need N % 128 == 0
])
def test_layer_validation(lib, fn, case, want):
    c = layer(**case)
    got = _call(lib, fn, FAKE, ctypes.byref(c), FAKE, 1)
    assert got == want


@pytest.mark.parametrize("fn", ["awq_gemv", "awq_gemm", "awq_gemv_gate_up", "awq_gemm_gate_up"])
def test_io_validation(lib, fn):
    c = layer()
    f = lambda x, cc, y, M: _call(lib, fn, x, cc, y, M)
    assert f(FAKE, None, FAKE, 1) == 1               # null layer
    assert f(None, ctypes.byref(c), FAKE, 1) == 1    # null x
    assert f(FAKE, ctypes.byref(c), None, 1) == 1    # null y
    assert f(FAKE, ctypes.byref(c), FAKE, -1) == 1   # negative M
    assert f(MISALIGNED, ctypes.byref(c), FAKE, 1) == 3
    assert f(FAKE, ctypes.byref(c), MISALIGNED, 1) == 3
    assert f(FAKE, ctypes.byref(c), FAKE, 1 << 30) == 2   # M*K beyond 2^31
    # M == 0 is an empty batch: success, nothing launched
    assert f(FAKE, ctypes.byref(c), FAKE, 0) == 0


def test_gemv_rejects_large_batches(lib):
    c = layer()
    assert lib.awq_gemv(FAKE, ctypes.byref(c), FAKE, 17, None, 0, None) == 4


def test_gemv_workspace(lib):
    """The GEMV reduces its K split inside each workgroup: the query is 0 for
    every shape, a NULL workspace is accepted, a misaligned one is not."""
    for M, K, N in ((1, 4096, 14336), (16, 4096, 28672), (1, 8192, 28672), (0, 8, 8)):
        assert lib.awq_gemv_workspace_bytes(M, K, N) == 0
    c = layer()
    assert lib.awq_gemv(FAKE, ctypes.byref(c), FAKE, 1, MISALIGNED, 64, None) == WS
    assert lib.awq_gemv(FAKE, ctypes.byref(c), FAKE, 0, None, 0, None) == 0


def test_status_enum_matches_header():
    """awq_status numbering as the header declares it: invalid value 1, shape 2,
    alignment 3, unsupported 4, workspace 5, HIP 6."""
    text = open(HEADER).read()
    body = re.search(r"typedef enum awq_status \{(.*?)\} awq_status;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    declared = {k: int(v) for k, v in re.findall(r"(AWQ_\w+)\s*=\s*(\d+)", body)}
    assert declared == {"AWQ_SUCCESS": 0, "AWQ_ERROR_INVALID_VALUE": 1, "AWQ_ERROR_SHAPE": 2,
                        "AWQ_ERROR_ALIGNMENT": 3, "AWQ_ERROR_UNSUPPORTED": 4,
                        "AWQ_ERROR_WORKSPACE": 5, "AWQ_ERROR_HIP": 6}
    for name, value in declared.items():
        assert getattr(binding, name) == value
        assert binding.STATUS_NAMES[value] == name


def test_gemm_gate_up_validation(lib):
    """Shapes the batched fused gate/up entry rejects before any launch."""
    f = lib.awq_gemm_gate_up
    assert f(FAKE, ctypes.byref(layer(N=24)), FAKE, 64, None) == 2                 # I not a multiple of 8
    assert f(FAKE, ctypes.byref(layer(K=128, G=32)), FAKE, 64, None) == 4          # G % 64
    assert f(FAKE, ctypes.byref(layer(K=384, G=128)), FAKE, 64, None) == 4         # K % 256
    assert f(FAKE, ctypes.byref(layer()), FAKE, 0, None) == 0                      # empty batch


def test_quantize_validation(lib):
    """Arguments the quantizer rejects before any launch."""
    f = lib.awq_quantize
    assert f(None, 128, 64, 128, 0, FAKE, FAKE, FAKE, None) == 1          # null w
    assert f(FAKE, 128, 64, 128, 0, FAKE, FAKE, None, None) == 1          # asymmetric needs qzeros
    assert f(FAKE, 0, 64, 128, 0, FAKE, FAKE, FAKE, None) == 1            # K = 0
    assert f(FAKE, 128, 64, 0, 1, FAKE, FAKE, None, None) == 1            # G = 0
    assert f(FAKE, 120, 64, 128, 1, FAKE, FAKE, None, None) == 2          # K % G
    assert f(FAKE, 128, 60, 128, 1, FAKE, FAKE, None, None) == 2          # N % 8
    assert f(FAKE, 128, 64, 12, 1, FAKE, FAKE, None, None) == 2           # G % 8
    assert f(MISALIGNED, 128, 64, 128, 1, FAKE, FAKE, None, None) == 3
    assert f(FAKE, 128, 64, 128, 0, FAKE, FAKE, MISALIGNED, None) == 3


def test_gate_up_validation(lib):
    """Shapes the fused gate/up entry rejects before any launch."""
    f = lib.awq_gemv_gate_up
    assert f(FAKE, ctypes.byref(layer(N=24)), FAKE, 1, None) == 2            # I not a multiple of 8
    assert f(FAKE, ctypes.byref(layer()), FAKE, 17, None) == 4               # batch above 16
    assert f(FAKE, ctypes.byref(layer(G=32)), FAKE, 1, None) == 4            # group not a multiple of 128
    # (any K: X that does not fit LDS is staged segment by segment)
    assert f(FAKE, ctypes.byref(layer()), FAKE, 0, None) == 0                # empty batch


def test_pack_validation(lib):
    assert lib.awq_pack(None, FAKE, 8, 8, None) == 1
    assert lib.awq_pack(FAKE, FAKE, 0, 8, None) == 1
    assert lib.awq_pack(FAKE, FAKE, 12, 8, None) == 2
    assert lib.awq_pack(FAKE, FAKE, 8, 12, None) == 2
    assert lib.awq_pack(MISALIGNED, FAKE, 8, 8, None) == 3
    assert lib.awq_pack_zeros(FAKE, None, 1, 8, None) == 1
    assert lib.awq_pack_zeros(FAKE, FAKE, 1, 4, None) == 2
    assert lib.awq_pack_zeros(FAKE, MISALIGNED, 1, 8, None) == 3


def test_dequant_validation(lib):
    c = layer()
    assert lib.awq_dequant(ctypes.byref(c), None, None) == 1
    assert lib.awq_dequant(ctypes.byref(c), MISALIGNED, None) == 3
    bad = layer(K=100)
    assert lib.awq_dequant(ctypes.byref(bad), FAKE, None) == 2


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        binding.load(str(tmp_path / "libawq.so"))


def test_scale_workspace_queries(lib):
    for fn in (lib.awq_channel_stats_workspace_bytes, lib.awq_scale_search_workspace_bytes):
        assert fn(64, 256, 128, 64) > 0
        assert fn(0, 256, 128, 64) == 0 and fn(64, 256, 128, 48) == 0
    # the search holds at least the migrated X, the candidate's packed weight,
    # the fp32 reference and the fp16 output (the migrated W is formed inside
    # the quantizer and never stored)
    need = 64 * 256 * 2 + 256 // 8 * 128 * 4 + 64 * 128 * 4 + 64 * 128 * 2
    assert lib.awq_scale_search_workspace_bytes(64, 256, 128, 64) >= need


def test_channel_stats_validation(lib):
    ws = lib.awq_channel_stats_workspace_bytes(64, 256, 128, 64)

    def call(x=FAKE, M=64, w=FAKE, K=256, N=128, G=64, xb=FAKE, wb=FAKE, wsp=FAKE, nb=ws):
        return lib.awq_channel_stats(x, M, w, K, N, G, xb, wb, wsp, nb, None)
    assert call(x=None) == 1 and call(M=0) == 1 and call(xb=None) == 1 and call(G=0) == 1
    assert call(K=260) == 2 and call(N=100) == 2 and call(G=48) == 2
    assert call(x=MISALIGNED) == 3 and call(w=MISALIGNED) == 3
    assert call(wsp=None) == WS and call(wsp=MISALIGNED) == WS and call(nb=ws - 1) == WS


def test_scale_search_validation(lib):
    ws = lib.awq_scale_search_workspace_bytes(64, 256, 128, 64)
    good = (ctypes.c_float * 3)(0.0, 0.5, 1.0)

    def call(x=FAKE, M=64, K=256, N=128, G=64, alphas=good, n=3, losses=FAKE, best=FAKE,
             wsp=FAKE, nb=ws):
        return lib.awq_scale_search(x, M, FAKE, K, N, G, 0, alphas, n, losses, best, None, wsp, nb,
                                    None)
    assert call(x=None) == 1 and call(M=-1) == 1 and call(losses=None) == 1 and call(best=None) == 1
    assert call(alphas=None) == 1 and call(n=0) == 1 and call(n=65) == 1
    for bad in (-0.1, 1.5, float("nan")):
        assert call(alphas=(ctypes.c_float * 1)(bad), n=1) == 1, bad
    assert call(K=260) == 2 and call(G=48) == 2
    assert call(M=1 << 20, K=4096) == 2          # M * K beyond 2^31
    assert call(x=MISALIGNED) == 3
    assert call(wsp=None) == WS and call(nb=ws - 1) == WS


def test_gemm_splitk_validation(lib):
    ws = lib.awq_gemm_splitk_workspace_bytes(64, 256, 4)
    assert ws == 4 * 64 * 256 * 4
    assert lib.awq_gemm_splitk_workspace_bytes(64, 256, 0) == 0
    assert lib.awq_gemm_splitk_workspace_bytes(64, 256, 17) == 0

    def call(M=64, splits=4, wsp=FAKE, nb=ws, **kw):
        lay = layer(K=1024, N=256, G=128, **kw)
        return lib.awq_gemm_splitk(FAKE, ctypes.byref(lay), FAKE, M, splits, wsp, nb, None)
    assert call(splits=0) == 1 and call(splits=17) == 1 and call(M=-1) == 1
    assert call(M=0) == 0                       # empty batch: nothing launched
    assert call(splits=3) == 4                  # 1024 / 3 is not whole
    assert call(splits=16) == 4                 # 64-k slices: less than a 128-k ring turn
    assert call(wsp=None) == WS and call(wsp=MISALIGNED) == WS and call(nb=ws - 1) == WS
    lay = layer(K=1024, N=256, G=256)
    assert lib.awq_gemm_splitk(FAKE, ctypes.byref(lay), FAKE, 64, 8, FAKE, 8 * 64 * 256 * 4,
                               None) == 4       # 128-k slices cut the 256-row groups


def test_gemm_splitk_static_validation(lib):
    """The no-allocation split-K rejects, before any launch, what awq_gemm_splitk
    rejects, and partial sums beyond its static scratch."""
    f = lib.awq_gemm_splitk_static
    lay = layer(K=1024, N=256, G=128)
    assert f(FAKE, ctypes.byref(lay), FAKE, 64, 0, None) == 1
    assert f(FAKE, ctypes.byref(lay), FAKE, 64, 17, None) == 1
    assert f(FAKE, ctypes.byref(lay), FAKE, -1, 4, None) == 1
    assert f(FAKE, ctypes.byref(lay), FAKE, 0, 4, None) == 0          # empty batch
    assert f(FAKE, ctypes.byref(lay), FAKE, 64, 3, None) == 4         # 1024 / 3 not whole
    assert f(MISALIGNED, ctypes.byref(lay), FAKE, 64, 4, None) == 3
    big = layer(K=4096, N=28672, G=128)
    scratch = binding.GEMM_SPLITK_STATIC_SCRATCH_BYTES
    assert 2 * 4096 * 28672 * 4 > scratch
    assert f(FAKE, ctypes.byref(big), FAKE, 4096, 2, None) == WS


def test_layout_struct_and_constants():
    """awq_layer ends with the layout field (a zeroed one is canonical); the
    header's layout values are the binding's."""
    assert ctypes.sizeof(binding.CLayer) == 40
    assert binding.CLayer.layout.offset == 36
    text = open(HEADER).read()
    assert re.search(r"#define AWQ_LAYOUT_CANONICAL 0\b", text)
    assert re.search(r"#define AWQ_LAYOUT_INTERLEAVED 1\b", text)
    assert re.search(r"#define AWQ_LAYOUT_BLOCKED 2\b", text)
    assert binding.LAYOUT_CANONICAL == 0 and binding.LAYOUT_INTERLEAVED == 1
    assert binding.LAYOUT_BLOCKED == 2


def test_repack_validation(lib):
    f = lib.awq_repack
    assert f(None, FAKE, 64, 64, 0, 1, None) == 1
    assert f(FAKE, None, 64, 64, 0, 1, None) == 1
    assert f(FAKE, FAKE, 0, 64, 0, 1, None) == 1
    assert f(FAKE, FAKE, 64, 64, 0, 3, None) == 1
    assert f(FAKE, FAKE, 64, 64, 3, 0, None) == 1
    other = FAKE + 0x1000000
    assert f(FAKE, other, 64, 64, 0, 2, None) == 2       # blocked words need N % 128 == 0
    assert f(FAKE, other, 64, 136, 2, 1, None) == 2
    assert f(FAKE, FAKE, 64, 128, 0, 2, None) == 1       # in place across the blocked layout
    assert f(FAKE, FAKE, 64, 128, 2, 1, None) == 1
    assert f(FAKE, FAKE, 64, 128, 2, 2, None) == 0       # same layout, in place: nothing to do
    assert f(FAKE, FAKE, 60, 64, 0, 1, None) == 2
    assert f(FAKE, FAKE, 64, 60, 0, 1, None) == 2
    assert f(FAKE, FAKE, 1 << 16, 1 << 16, 0, 1, None) == 2
    assert f(MISALIGNED, FAKE, 64, 64, 0, 1, None) == 3
    assert f(FAKE, FAKE, 64, 64, 1, 1, None) == 0          # same layout, in place: nothing to do


SYNC_CHILD = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from w4a16_group_quantized_amd import binding
lib = binding.load()
FAKE, MIS = 0x10000000, 0x10000002
c = binding.CLayer(FAKE, FAKE, FAKE, 128, 64, 128, 0)
bad = binding.CLayer(FAKE, FAKE, FAKE, 12, 64, 128, 0)
codes = [lib.awq_gemv(FAKE, ctypes.byref(c), FAKE, 17, None, 0, None),
         lib.awq_gemv(FAKE, ctypes.byref(bad), FAKE, 1, None, 0, None),
         lib.awq_gemm(MIS, ctypes.byref(c), FAKE, 1, None),
         lib.awq_gemm(FAKE, ctypes.byref(c), FAKE, 0, None),
         lib.awq_pack(None, FAKE, 8, 8, None)]
print(" ".join(str(v) for v in codes))
"""


@pytest.mark.parametrize("value", ["1", "yes"])
def test_sync_mode_keeps_validation(value):
    """AWQ_SYNC changes only what happens after a launch: rejected calls and
    empty batches return their codes with no HIP call (this host has no GPU)."""
    env = dict(os.environ, AWQ_SYNC=value)
    r = subprocess.run([sys.executable, "-c", SYNC_CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == ["4", "2", "3", "0", "1"]


def test_decode_sources_take_preloaded_arguments():
    """The decode kernels' sources, and only they, are built with kernarg
    preloading; the prefix still names existing sources."""
    from w4a16_group_quantized_amd import build as hip_build
    names = [os.path.basename(s) for s in hip_build.sources()]
    decode = [n for n in names if n.startswith("awq_gemv_stream_")]
    assert len(decode) >= 6
    for n in names:
        want = hip_build.KERNARG_PRELOAD if n in decode else []
        assert hip_build.source_flags(n, hip_build.SOURCE_FLAGS) == want, n
