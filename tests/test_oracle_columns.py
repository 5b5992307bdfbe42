"""The column-parallel forms of the oracle's layer (``linear_columns``,
``matmul_w_columns``) give bit-identical results to the single-threaded calls:
only the output columns are spread over host threads.  CPU only."""
import numpy as np
import pytest

from w4a16_group_quantized_amd import synth


@pytest.mark.parametrize("M,K,N,G,sym,threads", [
    (3, 256, 200, 64, False, 4), (1, 512, 1032, 128, True, 7), (5, 128, 16, 128, False, 16),
    (2, 64, 8, 8, False, 3),
])
def test_columns_bit_identical(oracle_lib, M, K, N, G, sym, threads):
    o = oracle_lib
    codes, zeros, scales = synth.make_layer(K, N, G, sym, 0.002, 0.02, 900 + K + N)
    X = synth.make_x(M, K, 900 + M)
    Q = o.pack(codes)
    QZ = None if sym else o.pack_zeros(zeros)
    y64, y16 = o.linear(X, Q, scales, QZ, G)
    c64, c16 = o.linear_columns(X, Q, scales, QZ, G, threads)
    assert np.array_equal(y64, c64) and np.array_equal(y16, c16)
    W = o.dequant(Q, scales, QZ, G)
    w64, w16 = o.matmul_w_columns(X, W, threads)
    assert np.array_equal(y64, w64) and np.array_equal(y16, w16)
