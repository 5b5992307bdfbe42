"""Seeded input generator: reproducibility and the published SplitMix64 values. CPU only."""
import numpy as np

from w4a16_group_quantized_amd import synth


def test_splitmix64_published_values():
    # First three outputs of SplitMix64 seeded with 0 (Steele, Lea and Flood 2014;
    # the values printed by the public reference implementation).
    got = [int(v) for v in synth.splitmix64(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_chunked_stream_equals_one_draw():
    s = synth.Stream(123)
    a = np.concatenate([s.raw(5), s.raw(7)])
    assert np.array_equal(a, synth.splitmix64(123, 0, 12))


def test_workload_inputs_deterministic_and_in_range():
    w = synth.WORKLOADS["tiny"]
    X1, c1, z1, s1 = synth.workload_inputs(w)
    X2, c2, z2, s2 = synth.workload_inputs(w)
    for a, b in [(X1, X2), (c1, c2), (z1, z2), (s1, s2)]:
        assert np.array_equal(a, b)
    assert X1.shape == (1, 512) and c1.shape == (512, 512)
    assert z1.shape == (4, 512) and s1.shape == (4, 512)
    assert c1.max() <= 15 and z1.max() <= 15
    sv = s1.view(np.float16).astype(np.float64)
    assert sv.min() >= np.float16(0.002) and sv.max() <= np.float16(0.02)
    # every code value appears with roughly equal frequency
    counts = np.bincount(c1.ravel(), minlength=16)
    assert counts.min() > 0.9 * c1.size / 16


def test_outlier_channels():
    w = synth.WORKLOADS["gate_up_m16"]
    ch = synth.outlier_channels(w.K, w.n_outliers, w.wid)
    assert len(ch) == 41 and len(set(ch.tolist())) == 41
    X = synth.make_x(2, w.K, w.wid, w.n_outliers, w.outlier_gain)
    Xp = synth.make_x(2, w.K, w.wid)
    xv, xp = X.view(np.float16).astype(np.float64), Xp.view(np.float16).astype(np.float64)
    assert np.array_equal(xv[:, ch], (xp[:, ch] * 20.0).astype(np.float16).astype(np.float64))
    rest = np.setdiff1d(np.arange(w.K), ch)
    assert np.array_equal(X[:, rest], Xp[:, rest])


def test_rows_are_prefix_stable():
    # the first row of an M-row draw is the M=1 draw (decode and batch share X's stream)
    a = synth.make_x(1, 1024, 9)
    b = synth.make_x(4, 1024, 9)
    assert np.array_equal(a[0], b[0])
