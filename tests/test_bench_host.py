"""bench.py's host logic on the CPU: the one-GPU guard, the algorithmic byte
counts, the counter-summary arithmetic (copy calibration, traffic per launch)
and the rule that traffic is reported only while the kernel's sources match the
summary.  Nothing here touches a GPU."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from w4a16_group_quantized_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,want", [
    # packed weight K N / 2 + scales 2 N K / G + zeros N K / (2 G) + X 2 M K + Y 2 M N
    ("decode_8b_gate", 30_543_872), ("gate_up_m16", 62_062_592), ("sym70b_m1", 117_571_584),
])
def test_algorithmic_bytes(name, want):
    w = synth.WORKLOADS[name]
    assert bench.alg_bytes(w, w.M) == want


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_summary_traffic_arithmetic(tmp_path, monkeypatch):
    """A copy of 64 MiB that reads half its bytes in FETCH_SIZE KiB (factor 2) and
    all of them in WRITE_SIZE (factor 1); a kernel with FETCH_SIZE 1000 KiB and
    WRITE_SIZE 10 KiB in every dispatch then moved 2 * 1000 + 10 KiB."""
    kern = "void awq::gemv::stream_kernel<4, 8, 16, 2, 1, false, true, 1, false>(...)"
    copy = "__amd_rocclr_copyBuffer"
    half = bench.CALIBRATION_COPY_BYTES / 1024 / 2
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write_counters(fetch, [{"Dispatch_Id": i, "Kernel_Name": kern, "Counter_Name": "FETCH_SIZE",
                             "Counter_Value": 1000.0} for i in range(20)] +
                    [{"Dispatch_Id": 100 + i, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE",
                      "Counter_Value": half} for i in range(5)])
    _write_counters(write, [{"Dispatch_Id": i, "Kernel_Name": kern, "Counter_Name": "WRITE_SIZE",
                             "Counter_Value": 10.0} for i in range(20)] +
                    [{"Dispatch_Id": 100 + i, "Kernel_Name": copy, "Counter_Name": "WRITE_SIZE",
                      "Counter_Value": 2 * half} for i in range(5)])
    out = str(tmp_path / "summary.txt")
    bench.summarize_pmc(out, [fetch, write], "gemv", ["a command"])
    text = open(out).read()
    assert "factor 2.0000" in text and "factor 1.0000" in text
    assert f"traffic_bytes_per_launch: {2 * 1000 * 1024 + 10 * 1024}" in text
    # the committed-traffic reader takes this file while the sources match it ...
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", out)
    assert bench.committed_traffic() == 2 * 1000 * 1024 + 10 * 1024
    # ... and reports nothing once they no longer do
    with open(out) as f:
        stale = f.read().replace(bench.source_hash("gemv"), "0" * 64)
    with open(out, "w") as f:
        f.write(stale)
    assert bench.committed_traffic() is None


def test_splitk_splits_rule():
    """The split-K slice count: up to 64 rows the measured rule (at least 512 k
    per slice, at most 448 workgroups of 64 x 256 up to 32 rows and 256 beyond),
    beyond 64 rows the cost model; only slice counts the layer allows."""
    from types import SimpleNamespace
    from w4a16_group_quantized_amd import binding

    def lay(K, N, G=128):
        return SimpleNamespace(K=K, N=N, group_size=G)
    assert binding.splitk_splits(16, lay(4096, 4096)) == 8        # 16 tiles, 512 k a slice
    assert binding.splitk_splits(16, lay(14336, 4096)) == 16      # 896 k a slice
    assert binding.splitk_splits(16, lay(4096, 28672)) == 4       # 448 workgroups
    assert binding.splitk_splits(64, lay(4096, 28672)) == 2       # 256 beyond 32 rows
    assert binding.splitk_splits(64, lay(4096, 14336)) == 4
    assert binding.splitk_splits(16, lay(1024, 4096)) == 2        # 512 k a slice at most 2
    assert binding.splitk_splits(16, lay(4096, 4096, 4096)) == 8  # one group per column
    assert binding.splitk_splits(16, lay(4096, 4096, 2048)) == 2  # slices of whole groups
    assert binding.splitk_splits(16, lay(3072, 4096, 1024)) == 1  # 1536 k: not whole groups
    assert binding.splitk_splits(16, lay(4096, 4096, 32)) == 8    # 32-k steps (G % 64 != 0)
    assert binding.splitk_splits(16, lay(4096, 4096, 16)) == 1    # the library splits no G = 16
    assert binding.splitk_splits(16, lay(4096, 4096, 8)) == 1
    for M in (96, 512, 2048):                                     # the cost model's range
        assert binding.splitk_splits(M, lay(4096, 4096)) in (1, 2, 4, 8, 16)
    assert binding.splitk_splits(2048, lay(4096, 4096)) == 1


def test_probe_library_exports():
    """The measurement probes (built by build()) load, every symbol resolved
    (bench.py loads them), and export the read and MFMA ceilings and the
    timeline probe's calls."""
    import ctypes
    import shutil
    import subprocess
    import probes
    if not os.path.exists(probes.LIBRARY) or shutil.which("nm") is None:
        pytest.skip("probes not built")
    ctypes.CDLL(probes.LIBRARY, mode=os.RTLD_NOW)
    out = subprocess.run(["nm", "-D", "--defined-only", probes.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    for name in ("awq_probe_stream_read", "awq_probe_mfma", "awq_timeline_gemv", "awq_timeline_gemm",
                 "awq_timeline_read", "awq_timeline_slots"):
        assert f" T {name}" in out, name
