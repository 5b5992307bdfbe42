"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only), run against every pin in a child process.

An out-of-bounds read or write, a signed overflow, a bad shift or a misaligned
access in oracle.c aborts the child with a sanitizer report, so a pin that
passes only because of what stray memory held cannot go unnoticed.  CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _libasan():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _libasan() is None,
                    reason="gcc with libasan is needed")
def test_pins_clean_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.dirname(oracle.SOURCE), oracle.SOURCE, "-o", so, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = _libasan()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), so],
                       capture_output=True, text=True, env=env, timeout=900)
    report = (r.stdout + r.stderr)[-3000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report
    assert r.returncode == 0, report
    assert r.stdout.strip().endswith("FAILED:"), report
