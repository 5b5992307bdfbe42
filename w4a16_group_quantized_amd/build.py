"""Builds libawq.so, the C-ABI library of HIP kernels for gfx950, in-tree.

    python -m w4a16_group_quantized_amd.build

Every HIP source under ``csrc/`` is compiled to an object in its own hipcc
process (in parallel) and the objects are linked into one shared library next
to this file.  Flags: -O3 for gfx950 only; no fast-math and no denormal
flushing (the dequantized weights must round exactly as IEEE fp16); packed-fp32
VALU instructions disabled; kernarg preloading for the decode kernels
(``SOURCE_FLAGS``).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libawq.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]

# Per-source flags, by file name prefix.  The decode kernels (one to four rows,
# awq_gemv_stream_*.hip) are built with kernarg preloading: gfx950 can hand a
# kernel its arguments in SGPRs at dispatch, so a wave starts computing
# addresses without first waiting on a scalar load of the argument block.  On
# the 4096 x 14336 decode layer a call went from 7.25 to 7.10 us; the 16-row
# kernels measured 1.3% slower with it and the GEMM unchanged, so they are
# built without it.
KERNARG_PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
SOURCE_FLAGS = {"awq_gemv_stream_": KERNARG_PRELOAD}


def source_flags(src: str, table: dict[str, list[str]]) -> list[str]:
    name = os.path.basename(src)
    return [f for prefix, flags in table.items() if name.startswith(prefix) for f in flags]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build(out: str = LIBRARY, extra_flags: list[str] | None = None, verbose: bool = False,
          srcs: list[str] | None = None, jobs: int | None = None,
          per_source: dict[str, list[str]] | None = None) -> str:
    """Compile every HIP source into ``out`` (always recompiles): each source to
    an object in its own hipcc process, in parallel, then one link.
    ``per_source`` maps file name prefixes to added flags (default: the
    library's ``SOURCE_FLAGS``)."""
    table = SOURCE_FLAGS if per_source is None else per_source
    srcs = srcs or sources()
    objdir = os.path.join(os.path.dirname(out), "_build", os.path.splitext(os.path.basename(out))[0])
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra_flags or [])
    objs = [os.path.join(objdir, os.path.splitext(os.path.basename(src))[0] + ".o") for src in srcs]
    jobs = jobs or min(len(srcs), max(1, min(os.cpu_count() or 1, 16)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, [hipcc(), *compile_flags, *source_flags(src, table), "-c", src, "-o", obj],
                             verbose)
                  for src, obj in zip(srcs, objs)]:
            f.result()
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
