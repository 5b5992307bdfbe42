"""Mutation check of the oracle's pins.

Each case plants one plausible mistake (a dropped term, a wrong sign, shift or
index, a transposed operand, a wrong rounding rule) in a copy of ``oracle.c``,
compiles the copy with the same flags, and runs every pin against it in a child
process.  Some pin must fail for every mistake; the real oracle must pass them
all (``test_oracle_pins.py``).  CPU only.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

# (name, text in oracle.c, replacement, which occurrence)
MUTANTS = [
    ("pack_nibble_order", "word |= c << (4 * j);", "word |= c << (4 * (7 - j));", 0),
    ("pack_zeros_nibble_order", "word |= z << (4 * j);", "word |= z << (4 * (7 - j));", 0),
    ("pack_no_mask", "codes[(size_t)(8 * r + j) * N + n] & 0xFu", "codes[(size_t)(8 * r + j) * N + n]", 0),
    ("unpack_code_shift", "(word >> (4 * (k % 8)))", "(word >> (4 * (7 - k % 8)))", 0),
    ("unpack_code_row", "Q[(size_t)(k / 8) * N + n]", "Q[(size_t)(k / 16) * N + n]", 0),
    ("zero_word_index", "QZ[(size_t)g * (N / 8) + n / 8]", "QZ[(size_t)g * (N / 8) + n % (N / 8)]", 0),
    ("zero_nibble_shift", "(word >> (4 * (n % 8)))", "(word >> (4 * ((n / 8) % 8)))", 0),
    ("symmetric_zero_7", "if (QZ == NULL) return 8;", "if (QZ == NULL) return 7;", 0),
    ("group_interleaved", "int g = k / G;", "int g = k % (K / G);", 0),
    ("scales_transposed", "uint16_t s = S[(size_t)g * N + n];", "uint16_t s = S[(size_t)n * (K / G) + g];", 0),
    ("dequant_sign", "(double)(q - z) * oracle_h2d(s)", "(double)(z - q) * oracle_h2d(s)", 0),
    ("dequant_prescaled_zero", "oracle_d2h((double)(q - z) * oracle_h2d(s))",
     "oracle_d2h(oracle_h2d(oracle_d2h(q * oracle_h2d(s))) - oracle_h2d(oracle_d2h(z * oracle_h2d(s))))", 0),
    ("d2h_ties_away", "(frac == 0.5 && fmod(fl, 2.0) != 0.0)", "(frac == 0.5)", 0),
    ("d2h_truncate", "r = fl + 1.0;", "r = fl;", 0),
    ("d2h_no_subnormal_clamp", "int Eq = E < -14 ? -14 : E;", "int Eq = E;", 0),
    ("d2h_overflow_threshold", "if (a >= 65520.0)", "if (a > 65504.0)", 0),
    ("h2d_bias", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)", 0),
    ("h2d_subnormal_scale", "ldexp((double)f, -24)", "ldexp((double)f, -25)", 0),
    ("matmul_drop_first_k", "for (int k = 0; k < K; ++k) {\n            double x", "for (int k = 1; k < K; ++k) {\n            double x", 0),
    ("matmul_drop_last_k", "for (int k = 0; k < K; ++k) {\n            double x", "for (int k = 0; k < K - 1; ++k) {\n            double x", 0),
    ("matmul_x_transposed", "X[(size_t)m * K + k]", "X[(size_t)k * M + m]", 0),
    ("matmul_w_transposed", "acc[n] += x * wrow[n];", "acc[n] += x * Wd[((size_t)n * K + k) % ((size_t)K * N)];", 0),
    ("matmul_fp32_accumulate", "acc[n] += x * wrow[n];", "acc[n] = (float)(acc[n] + x * wrow[n]);", 0),
    ("matmul_y_row_offset", "Y16[(size_t)m * N + n] = oracle_d2h(acc[n]);", "Y16[(size_t)m * N + n] = oracle_d2h(acc[(n + 1) % N]);", 0),
    ("quant_range_16", "r = range / 15.0;", "r = range / 16.0;", 0),
    ("quant_sym_8", "r = (double)amax / 7.0;", "r = (double)amax / 8.0;", 0),
    # the scale's range or quotient formed in fp32 before the fp16 rounding
    ("quant_range_fp32", "double range = (double)hi - (double)lo;", "double range = (double)(hi - lo);", 0),
    ("quant_quotient_fp32", "r = range / 15.0;", "r = (double)((float)range / 15.0f);", 0),
    ("quant_zero_sign", "z = clamp_code(rintf(-lo / sv));", "z = clamp_code(rintf(lo / sv));", 0),
    ("quant_truncate", "clamp_code(rintf(w / sv) + z)", "clamp_code(truncf(w / sv) + z)", 0),
    ("quant_no_clamp_low", "return v < 0.0f ? 0.0f : (v > 15.0f ? 15.0f : v);", "return v > 15.0f ? 15.0f : v;", 0),
    ("quant_group_rows", "for (int k = g * G; k < (g + 1) * G; ++k) {\n                float w = (float)oracle_h2d(W[(size_t)k * N + n]);\n                if (w < lo)", "for (int k = g * G; k < (g + 1) * G - 1; ++k) {\n                float w = (float)oracle_h2d(W[(size_t)k * N + n]);\n                if (w < lo)", 0),
    ("interleave_order", "static int interleaved_nibble(int j) { return 4 * (j % 2) + j / 2; }",
     "static int interleaved_nibble(int j) { return 2 * (j % 4) + j / 4; }", 0),
    ("deinterleave_as_interleave", "o |= ((w >> (4 * interleaved_nibble(j))) & 0xFu) << (4 * j);",
     "o |= ((w >> (4 * j)) & 0xFu) << (4 * interleaved_nibble(j));", 0),
    ("block_rows_columns_swapped",
     "out[(size_t)(n / 128) * R * 128 + (size_t)r * 128 + n % 128] = Q[(size_t)r * N + n];",
     "out[(size_t)(n / 128) * R * 128 + (size_t)(n % 128) * R + r] = Q[(size_t)r * N + n];", 0),
    ("block_stride_N",
     "out[(size_t)(n / 128) * R * 128 + (size_t)r * 128 + n % 128] = Q[(size_t)r * N + n];",
     "out[(size_t)(n / 128) * 128 + (size_t)r * N + n % 128] = Q[(size_t)r * N + n];", 0),
    ("silu_is_sigmoid", "return t / (1.0 + exp(-t));", "return 1.0 / (1.0 + exp(-t));", 0),
    ("silu_exp_sign", "return t / (1.0 + exp(-t));", "return t / (1.0 + exp(t));", 0),
    ("gate_up_swapped", "oracle_silu(row[n]) * row[I + n]", "oracle_silu(row[I + n]) * row[n]", 0),
    ("gate_up_no_silu", "oracle_silu(row[n]) * row[I + n]", "row[n] * row[I + n]", 0),
    ("gate_up_row_stride", "const double *row = Y64 + (size_t)m * 2 * I;", "const double *row = Y64 + (size_t)m * I;", 0),
    ("stats_x_no_abs", "sum += fabs(oracle_h2d(X[(size_t)m * K + k]));", "sum += oracle_h2d(X[(size_t)m * K + k]);", 0),
    ("stats_w_not_normalized", "wbar[k] += fabs(oracle_h2d(W[(size_t)k * N + n])) / a;", "wbar[k] += fabs(oracle_h2d(W[(size_t)k * N + n]));", 0),
    ("stats_w_mean_over_k", "for (int k = 0; k < K; ++k) wbar[k] /= N;", "for (int k = 0; k < K; ++k) wbar[k] /= K;", 0),
    ("stats_w_group_off_by_one", "for (int k = g * G; k < (g + 1) * G; ++k) {\n                double v", "for (int k = g * G; k < (g + 1) * G - 1; ++k) {\n                double v", 0),
    ("candidate_exponents_swapped", "c[k] = pow(xa, alpha) / pow(wa, 1.0 - alpha);", "c[k] = pow(xa, 1.0 - alpha) / pow(wa, alpha);", 0),
    ("candidate_no_floor", "double xa = xbar[k] > 1e-4 ? xbar[k] : 1e-4;", "double xa = xbar[k];", 0),
    ("migrate_x_times_c", "oracle_d2h(oracle_h2d(X[(size_t)m * K + k]) / c[k])", "oracle_d2h(oracle_h2d(X[(size_t)m * K + k]) * c[k])", 0),
    ("migrate_w_divided", "oracle_d2h(c[k] * oracle_h2d(W[(size_t)k * N + n]))", "oracle_d2h(oracle_h2d(W[(size_t)k * N + n]) / c[k])", 0),
    ("loss_unrounded_output", "double d = Yr[i] - oracle_h2d(Yh16[i]);", "double d = Yr[i] - Yh[i];", 0),
    ("loss_reference_quantized", "oracle_matmul_w(X, W, M, K, N, Yr, Yr16);", "oracle_matmul_w(Xs, Wq, M, K, N, Yr, Yr16);", 0),
    ("search_last_minimum", "if (best < 0 || losses[i] < losses[best]) best = i;", "if (best < 0 || losses[i] <= losses[best]) best = i;", 0),
]


def _mutate(src, old, new, occurrence):
    assert src.count(old) >= occurrence + 1, old
    idx = -1
    for _ in range(occurrence + 1):
        idx = src.index(old, idx + 1)
    return src[:idx] + new + src[idx + len(old):]


def _run_mutant(tmp, case):
    name, old, new, occ = case
    src = open(oracle.SOURCE).read()
    mutated = _mutate(src, old, new, occ)
    c_path = os.path.join(tmp, f"{name}.c")
    with open(c_path, "w") as f:
        f.write(mutated)
    so = oracle.build(c_path, os.path.join(tmp, f"{name}.so"))
    pins = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_pins.py")
    r = subprocess.run([sys.executable, pins, so], capture_output=True, text=True, timeout=300)
    return name, r.returncode, r.stdout.strip()[-300:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=6) as ex:
        results = list(ex.map(lambda c: _run_mutant(str(tmp_path), c), MUTANTS))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, f"planted mistakes no pin caught: {survivors}"
