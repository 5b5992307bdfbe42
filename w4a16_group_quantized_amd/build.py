"""Builds libawq.so, the C-ABI library of HIP kernels for gfx950, in-tree.

    python -m w4a16_group_quantized_amd.build

Every HIP source under ``csrc/`` goes into one shared library next to this
file.  The measurement probes under ``probes/`` (a plain streaming read and an
MFMA rate probe, used only by bench.py) go into ``probes/libawq_probes.so``.  Flags: -O3 for gfx950 only; no fast-math and no denormal flushing (the
dequantized weights must round exactly as IEEE fp16); packed-fp32 VALU
instructions disabled.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libawq.so")
PROBES = os.path.join(HERE, "probes")
PROBE_LIBRARY = os.path.join(PROBES, "libawq_probes.so")
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


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIBRARY, extra_flags: list[str] | None = None, verbose: bool = False,
          srcs: list[str] | None = None) -> str:
    """Compile every HIP source into ``out`` (always recompiles)."""
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *(srcs or sources()), "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)
    return out


def build_probes(verbose: bool = False) -> str:
    """Compile the measurement probes into ``probes/libawq_probes.so``."""
    return build(PROBE_LIBRARY, verbose=verbose,
                 srcs=sorted(glob.glob(os.path.join(PROBES, "*.hip"))))


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probes(verbose=True))
