"""Measurement probes: a plain streaming read and an MFMA rate probe
(``ceilings.hip``, used by bench.py), and the timeline probe (``timeline.hip``:
the library's decode GEMV and prefill GEMM kernels compiled with per-wave
timestamps), built into ``libawq_probes.so`` here.

They measure what this GPU sustains on the two bound resources (HBM reads and
fp16 matrix-core chains), and where a call's time goes.  They are not part of
the library and nothing in it loads them.

    python -m probes                    # build
    python -m probes timeline [--out FILE]
"""
from __future__ import annotations

import glob
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libawq_probes.so")


def build(verbose: bool = False) -> str:
    """Compile the probes with the library's hipcc flags (always recompiles).
    The read probe takes its arguments preloaded in SGPRs, as the library's
    decode kernels do, so that the floor it measures has the same start-up; the
    timeline probe's kernels are built without, like the library's other
    kernels (its decode kernel's calls then run about 0.15 us longer than the
    library's)."""
    from w4a16_group_quantized_amd import build as hip_build
    return hip_build.build(LIBRARY, verbose=verbose,
                           srcs=sorted(glob.glob(os.path.join(HERE, "*.hip"))),
                           per_source={"ceilings": hip_build.KERNARG_PRELOAD})

