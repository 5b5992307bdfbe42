/*
 * Plain CPU oracle for the W4A16 group-quantized linear layer (AWQ inference).
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists to check the HIP library; it is
 * never part of the product path.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table or
 * helper with the HIP sources, and it includes nothing from them.
 *
 * What it computes, and where that comes from:
 *   - AWQ keeps weights as 4-bit codes, eight of them inside one INT32 word,
 *     with floating-point scales and zero points shared by groups of 128
 *     weights (mbrenndoerfer.com, "AWQ > Implementation", section
 *     "Understanding the Quantization Structure"; pyshine.com AutoAWQ tour,
 *     "From Install to Your First Model": zero_point / q_group_size / w_bit).
 *   - Symmetric dequantization is weight = scale[o] * (code - 8), codes 0..15,
 *     8 being the symmetric zero point (fak explainer, "Format Specification >
 *     Dequantization Formula").
 *   - The kernels dequantize on the fly inside the matrix multiplication and do
 *     fp16 arithmetic on activations (unfragile.ai AutoAWQ page, the WQLinear
 *     paragraph; mbrenndoerfer.com, "Loading and Using AWQ Models").
 *
 *   - The fused inference stack merges a layer's gate and up projections into
 *     one concatenated MLP module (pyshine.com AutoAWQ tour, the introduction
 *     and "The Quantization Flow Up Close": QuantFusedMLP); the models it
 *     serves are Llama-family (unfragile.ai AutoAWQ page, the Llama/Mistral
 *     paragraph), whose MLP multiplies SiLU(gate) by up.
 *
 * Readings taken where the pages are silent (each one is a plain choice that
 * the rest of the pages support):
 *   R1  nibble order: code j of a word sits in bits 4j..4j+3 (least significant
 *       nibble first).
 *   R2  packed axis: the eight codes of one word are eight consecutive k of one
 *       output column n, so the packed weight is Q[K/8][N].
 *   R3  group axis: G consecutive k share one scale and one zero for each
 *       column n, group index g = k / G; scales are S[K/G][N].
 *   R4  zero points are 4-bit integers 0..15, packed eight per word along n:
 *       QZ[K/G][N/8]; no zero tensor means the symmetric zero 8.
 *   R5  asymmetric dequant w = fp16(s * (q - z)): the integer difference is
 *       exact, then one multiply and one round-to-nearest-even to fp16.
 *   R6  the layer output is Y = X * W with W[K][N] the dequantized fp16 weight,
 *       accumulated exactly enough (here fp64, increasing k) and rounded once
 *       to fp16.
 *   R7  fp16 is IEEE 754 binary16: subnormals kept, overflow to infinity,
 *       round to nearest, ties to even.
 *   R8-R11 (codes above 15 masked when packed; K, N and G multiples of 8 and
 *       K of G; the synthetic inputs' outlier channels and fp16 draws) concern
 *       the callers and the input generator, not the arithmetic here.
 *   R13 quantizer (the step before the layer): each group of G weights of a
 *       column is rounded to integer levels against a scale and zero point
 *       (pyshine.com AutoAWQ tour, "The Quantization Flow Up Close": the
 *       pseudo-quantization pass; "From Install to Your First Model":
 *       zero_point, q_group_size, w_bit).  The pages give no formula; this is
 *       textbook min-max:
 *         asymmetric: r = hi - lo (r = |hi| if hi == lo), s = fp16(r / 15),
 *                     z = clamp(rint(-lo / s), 0, 15)
 *         symmetric:  r = max |w|, s = fp16(r / 7), z = 8
 *         both:       s = 1 if it rounds to 0; q = clamp(rint(w / s) + z, 0, 15)
 *       with lo, hi the group's minimum and maximum.  The scale is the exact
 *       real r / 15 (or r / 7) rounded once to fp16.  The two decisions that
 *       yield integers (z and q) are taken in fp32 (IEEE, round to nearest
 *       even), the precision the GPU kernel decides them in.
 *   R17 kernel-private layout (the step after packing, for faster kernels):
 *       the code of k = 8r + j moves to nibble 4 (j % 2) + j / 2 of the same
 *       word: even k in the low half-word, odd k in the high half-word.  The
 *       pages name private packing formats (GEMVFast, Marlin) without giving
 *       one; oracle_interleave / oracle_deinterleave are that permutation and
 *       its inverse.
 *   R18 kernel-private blocked layout: the interleaved words, moved so that
 *       each run of 128 columns holds all K/8 packed rows together: word
 *       [r][n] goes to index (n / 128) * (K/8) * 128 + r * 128 + n % 128
 *       (N % 128 == 0).  Same reading as R17: the pages name private formats
 *       without giving one.  oracle_block / oracle_unblock move the words
 *       (nibbles untouched); the blocked layout is oracle_block of the
 *       interleaved words.
 *   R12 fused gate/up: the layer's N = 2I columns are [gate | up]; the output
 *       is h[m][n] = fp16(SiLU(y(m, n)) * y(m, I + n)), n < I, with y the
 *       layer's exact (unrounded) sums and SiLU(t) = t / (1 + e^-t), rounded
 *       once.
 *   R14 channel statistics of the scale search (pyshine.com AutoAWQ tour, "The
 *       Quantization Flow Up Close": a per-channel mean of normalized weights
 *       and a mean of activations; the AwqQuantizer captures activation
 *       magnitudes): for input channel k,
 *         xbar[k] = mean over the calibration rows m of |x(m, k)|,
 *         wbar[k] = mean over the output columns n of |w(k, n)| / a(g, n),
 *       with a(g, n) the largest |w| of k's quantization group in column n
 *       (normalized per group: the pages do not say over what; a column whose
 *       group is all zero adds 0).
 *   R15 candidate scales (same passages; "duo_scaling" uses both statistics,
 *       and the scales come from a grid search): for a grid value alpha in
 *       [0, 1], c[k] = max(xbar[k], 1e-4)^alpha / max(wbar[k], 1e-4)^(1 - alpha).
 *       The grid itself is the caller's; the floor keeps c finite and nonzero.
 *   R16 objective (same passages: the FP16 module is run once as a reference
 *       and the candidate that minimizes the output error is kept; dividing
 *       the preceding op's output by c and multiplying the weights by c is
 *       invisible before rounding, "scale_ln_fcs"): the migrated inputs are
 *       X'(m, k) = fp16(x(m, k) / c[k]) and W'(k, n) = fp16(c[k] * w(k, n)),
 *       each rounded once; W' is quantized by R13 and dequantized by R5; the
 *       candidate's output is Y' = fp16(X' * deq(W')) (R6); the loss is the
 *       mean over (m, n) of (y - y')^2 with y the exact X * W.  The search
 *       keeps the first grid value of least loss.
 *
 * Everything is single threaded, unblocked and written for reading, not speed.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* IEEE 754 binary16 codec (R7): 1 sign bit, 5 exponent bits with bias 15,   */
/* 10 fraction bits.                                                          */
/* ------------------------------------------------------------------------- */

double oracle_h2d(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);            /* subnormal (or zero): f * 2^-24 */
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

uint16_t oracle_d2h(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00);
    /* 65504 is the largest finite half; halfway to 65536 (65520) ties to the
     * even neighbour, which is 65536 and therefore infinity. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00);
    if (a == 0.0) return sign;

    int e2;
    frexp(a, &e2);           /* a = m * 2^e2 with 0.5 <= m < 1 */
    int E = e2 - 1;          /* a in [2^E, 2^(E+1)) */
    int Eq = E < -14 ? -14 : E; /* below 2^-14 the spacing stays 2^-24 */
    double n = ldexp(a, 10 - Eq); /* a measured in units of the half spacing */
    double fl = floor(n);
    double frac = n - fl;
    double r = fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;

    uint32_t bits;
    if (E < -14) {
        bits = (uint32_t)r;  /* subnormal; r == 1024 lands on the smallest normal */
    } else {
        /* r in [1024, 2048]; r == 2048 carries into the exponent field */
        bits = ((uint32_t)(E + 15) << 10) + (uint32_t)r - 1024u;
    }
    return (uint16_t)(sign | bits);
}

void oracle_h2d_n(const uint16_t *h, size_t count, double *out)
{
    for (size_t i = 0; i < count; ++i) out[i] = oracle_h2d(h[i]);
}

void oracle_d2h_n(const double *x, size_t count, uint16_t *out)
{
    for (size_t i = 0; i < count; ++i) out[i] = oracle_d2h(x[i]);
}

/* ------------------------------------------------------------------------- */
/* Packing (R1, R2, R4): eight 4-bit codes per 32-bit word.                   */
/* ------------------------------------------------------------------------- */

void oracle_pack(const uint8_t *codes, int K, int N, int32_t *Q)
{
    for (int r = 0; r < K / 8; ++r) {
        for (int n = 0; n < N; ++n) {
            uint32_t word = 0;
            for (int j = 0; j < 8; ++j) {
                uint32_t c = codes[(size_t)(8 * r + j) * N + n] & 0xFu;
                word |= c << (4 * j);
            }
            Q[(size_t)r * N + n] = (int32_t)word;
        }
    }
}

void oracle_pack_zeros(const uint8_t *zeros, int groups, int N, int32_t *QZ)
{
    for (int g = 0; g < groups; ++g) {
        for (int c = 0; c < N / 8; ++c) {
            uint32_t word = 0;
            for (int j = 0; j < 8; ++j) {
                uint32_t z = zeros[(size_t)g * N + 8 * c + j] & 0xFu;
                word |= z << (4 * j);
            }
            QZ[(size_t)g * (N / 8) + c] = (int32_t)word;
        }
    }
}

int oracle_code(const int32_t *Q, int N, int k, int n)
{
    uint32_t word = (uint32_t)Q[(size_t)(k / 8) * N + n];
    return (int)((word >> (4 * (k % 8))) & 0xFu);
}

int oracle_zero(const int32_t *QZ, int N, int g, int n)
{
    if (QZ == NULL) return 8; /* symmetric zero point */
    uint32_t word = (uint32_t)QZ[(size_t)g * (N / 8) + n / 8];
    return (int)((word >> (4 * (n % 8))) & 0xFu);
}

void oracle_unpack(const int32_t *Q, int K, int N, uint8_t *codes)
{
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            codes[(size_t)k * N + n] = (uint8_t)oracle_code(Q, N, k, n);
}

void oracle_unpack_zeros(const int32_t *QZ, int groups, int N, uint8_t *zeros)
{
    for (int g = 0; g < groups; ++g)
        for (int n = 0; n < N; ++n)
            zeros[(size_t)g * N + n] = (uint8_t)oracle_zero(QZ, N, g, n);
}

/* ------------------------------------------------------------------------- */
/* Kernel-private layout (R17): the same words, nibbles reordered inside each  */
/* word.  The pages name packing formats private to faster kernels (GEMVFast,  */
/* Marlin; unpack_reorder_pack repacks bits for another runtime: pyshine.com   */
/* AutoAWQ tour, "The Quantization Flow Up Close") without giving one; the     */
/* reading here: the code of k = 8r + j sits at nibble 4 (j % 2) + j / 2 of    */
/* word [r][n], i.e. the four even k in the low half-word (k 0, 2, 4, 6 at     */
/* nibbles 0..3) and the four odd k in the high half-word (nibbles 4..7).      */
/* ------------------------------------------------------------------------- */

static int interleaved_nibble(int j) { return 4 * (j % 2) + j / 2; }

void oracle_interleave(const int32_t *Q, int K, int N, int32_t *out)
{
    for (size_t i = 0; i < (size_t)(K / 8) * N; ++i) {
        uint32_t w = (uint32_t)Q[i], o = 0;
        for (int j = 0; j < 8; ++j)
            o |= ((w >> (4 * j)) & 0xFu) << (4 * interleaved_nibble(j));
        out[i] = (int32_t)o;
    }
}

void oracle_deinterleave(const int32_t *Q, int K, int N, int32_t *out)
{
    for (size_t i = 0; i < (size_t)(K / 8) * N; ++i) {
        uint32_t w = (uint32_t)Q[i], o = 0;
        for (int j = 0; j < 8; ++j)
            o |= ((w >> (4 * interleaved_nibble(j))) & 0xFu) << (4 * j);
        out[i] = (int32_t)o;
    }
}

/* R18: word (r, n) of a [K/8][N] array to its place in 128-column blocks.    */
void oracle_block(const int32_t *Q, int K, int N, int32_t *out)
{
    const int R = K / 8;
    for (int r = 0; r < R; ++r)
        for (int n = 0; n < N; ++n)
            out[(size_t)(n / 128) * R * 128 + (size_t)r * 128 + n % 128] = Q[(size_t)r * N + n];
}

void oracle_unblock(const int32_t *B, int K, int N, int32_t *out)
{
    const int R = K / 8;
    for (int r = 0; r < R; ++r)
        for (int n = 0; n < N; ++n)
            out[(size_t)r * N + n] = B[(size_t)(n / 128) * R * 128 + (size_t)r * 128 + n % 128];
}

/* ------------------------------------------------------------------------- */
/* Dequantization (R3, R5, and the symmetric formula of the fak explainer).   */
/* ------------------------------------------------------------------------- */

uint16_t oracle_dequant_one(int q, int z, uint16_t s)
{
    /* (q - z) is a small integer and s has 11 significant bits, so the double
     * product is exact; the only rounding is the final conversion to fp16. */
    return oracle_d2h((double)(q - z) * oracle_h2d(s));
}

void oracle_dequant(const int32_t *Q, const uint16_t *S, const int32_t *QZ,
                    int K, int N, int G, uint16_t *W)
{
    for (int k = 0; k < K; ++k) {
        int g = k / G;
        for (int n = 0; n < N; ++n) {
            int q = oracle_code(Q, N, k, n);
            int z = oracle_zero(QZ, N, g, n);
            uint16_t s = S[(size_t)g * N + n];
            W[(size_t)k * N + n] = oracle_dequant_one(q, z, s);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* The layer (R6): Y[M][N] = X[M][K] * W[K][N].                                */
/* ------------------------------------------------------------------------- */

void oracle_matmul_w(const uint16_t *X, const uint16_t *W, int M, int K, int N,
                     double *Y64, uint16_t *Y16)
{
    /* Every product of two halves is exact in double.  Each output is summed
     * over k in increasing order; the loop over n sits innermost only so that
     * W is walked row by row, which leaves each output's order unchanged.
     * W is decoded to double once (the decoding is exact). */
    double *Wd = (double *)malloc((size_t)K * N * sizeof(double));
    double *acc = (double *)malloc((size_t)N * sizeof(double));
    for (size_t i = 0; i < (size_t)K * N; ++i) Wd[i] = oracle_h2d(W[i]);
    for (int m = 0; m < M; ++m) {
        for (int n = 0; n < N; ++n) acc[n] = 0.0;
        for (int k = 0; k < K; ++k) {
            double x = oracle_h2d(X[(size_t)m * K + k]);
            const double *wrow = Wd + (size_t)k * N;
            for (int n = 0; n < N; ++n) acc[n] += x * wrow[n];
        }
        for (int n = 0; n < N; ++n) {
            if (Y64) Y64[(size_t)m * N + n] = acc[n];
            if (Y16) Y16[(size_t)m * N + n] = oracle_d2h(acc[n]);
        }
    }
    free(acc);
    free(Wd);
}

int oracle_linear(const uint16_t *X, const int32_t *Q, const uint16_t *S,
                  const int32_t *QZ, int M, int K, int N, int G,
                  double *Y64, uint16_t *Y16)
{
    uint16_t *W = (uint16_t *)malloc((size_t)K * N * sizeof(uint16_t));
    if (W == NULL) return -1;
    oracle_dequant(Q, S, QZ, K, N, G, W);
    oracle_matmul_w(X, W, M, K, N, Y64, Y16);
    free(W);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Fused gate/up epilogue (R12).                                              */
/* ------------------------------------------------------------------------- */

double oracle_silu(double t)
{
    /* t * sigmoid(t); for t far below zero exp(-t) overflows to infinity and
     * the quotient is the correctly signed zero. */
    return t / (1.0 + exp(-t));
}

void oracle_gate_up(const double *Y64, int M, int I, uint16_t *H16)
{
    for (int m = 0; m < M; ++m) {
        const double *row = Y64 + (size_t)m * 2 * I;
        for (int n = 0; n < I; ++n)
            H16[(size_t)m * I + n] = oracle_d2h(oracle_silu(row[n]) * row[I + n]);
    }
}

/* ------------------------------------------------------------------------- */
/* Quantizer (R13).                                                          */
/*                                                                           */
/* Scale: the group's extremes are fp16 values, so hi - lo is exact in       */
/* double (two halves span at most 2^-24 .. 2^16, 40 bits < 53).  The double */
/* quotient range / 15 then rounds to fp16 exactly as the real quotient      */
/* would: the real quotient either equals an fp16 rounding midpoint m (then */
/* m, with 12 significant bits, is a double and the correctly rounded double */
/* quotient is m itself) or lies at least 2^-42 |q| away from every midpoint (range - 15 m */
/* is a nonzero multiple of the smaller of their lowest bits), far beyond    */
/* the double's 2^-53 relative error.  The same holds for max|w| / 7.  So    */
/* oracle_d2h of the double quotient is the exact scale rounded once.        */
/*                                                                           */
/* Codes and zero points: float arithmetic is IEEE single precision here     */
/* (SSE, no contraction), the precision the GPU kernel decides them in.      */
/* ------------------------------------------------------------------------- */

static float clamp_code(float v)
{
    return v < 0.0f ? 0.0f : (v > 15.0f ? 15.0f : v);
}

void oracle_quantize(const uint16_t *W, int K, int N, int G, int symmetric,
                     uint8_t *codes, uint16_t *S, uint8_t *zeros)
{
    for (int g = 0; g < K / G; ++g) {
        for (int n = 0; n < N; ++n) {
            float lo = INFINITY, hi = -INFINITY, amax = 0.0f;
            for (int k = g * G; k < (g + 1) * G; ++k) {
                float w = (float)oracle_h2d(W[(size_t)k * N + n]);
                if (w < lo) lo = w;
                if (w > hi) hi = w;
                if (fabsf(w) > amax) amax = fabsf(w);
            }
            double r;
            float z;
            if (symmetric) {
                r = (double)amax / 7.0;
                z = 8.0f;
            } else {
                double range = (double)hi - (double)lo;
                if (range == 0.0) range = fabs((double)hi);
                r = range / 15.0;
            }
            uint16_t sh = oracle_d2h(r);
            if ((sh & 0x7FFF) == 0) sh = 0x3C00;            /* 1.0 */
            float sv = (float)oracle_h2d(sh);
            if (!symmetric) z = clamp_code(rintf(-lo / sv));
            S[(size_t)g * N + n] = sh;
            if (zeros) zeros[(size_t)g * N + n] = (uint8_t)z;
            for (int k = g * G; k < (g + 1) * G; ++k) {
                float w = (float)oracle_h2d(W[(size_t)k * N + n]);
                codes[(size_t)k * N + n] = (uint8_t)clamp_code(rintf(w / sv) + z);
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Scale migration and its search objective (R14, R15, R16).                  */
/* ------------------------------------------------------------------------- */

void oracle_channel_stats(const uint16_t *X, int M, const uint16_t *W, int K, int N, int G,
                          double *xbar, double *wbar)
{
    for (int k = 0; k < K; ++k) {
        double sum = 0.0;
        for (int m = 0; m < M; ++m) sum += fabs(oracle_h2d(X[(size_t)m * K + k]));
        xbar[k] = sum / M;
    }
    for (int k = 0; k < K; ++k) wbar[k] = 0.0;
    for (int n = 0; n < N; ++n) {
        for (int g = 0; g < K / G; ++g) {
            double a = 0.0;
            for (int k = g * G; k < (g + 1) * G; ++k) {
                double v = fabs(oracle_h2d(W[(size_t)k * N + n]));
                if (v > a) a = v;
            }
            if (a == 0.0) continue;
            for (int k = g * G; k < (g + 1) * G; ++k)
                wbar[k] += fabs(oracle_h2d(W[(size_t)k * N + n])) / a;
        }
    }
    for (int k = 0; k < K; ++k) wbar[k] /= N;
}

void oracle_scale_candidate(const double *xbar, const double *wbar, int K, double alpha, double *c)
{
    for (int k = 0; k < K; ++k) {
        double xa = xbar[k] > 1e-4 ? xbar[k] : 1e-4;
        double wa = wbar[k] > 1e-4 ? wbar[k] : 1e-4;
        c[k] = pow(xa, alpha) / pow(wa, 1.0 - alpha);
    }
}

void oracle_migrate(const uint16_t *X, const uint16_t *W, int M, int K, int N, const double *c,
                    uint16_t *Xs, uint16_t *Ws)
{
    for (int m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k)
            Xs[(size_t)m * K + k] = oracle_d2h(oracle_h2d(X[(size_t)m * K + k]) / c[k]);
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            Ws[(size_t)k * N + n] = oracle_d2h(c[k] * oracle_h2d(W[(size_t)k * N + n]));
}

int oracle_scale_loss(const uint16_t *X, const uint16_t *W, int M, int K, int N, int G,
                      int symmetric, const double *c, double *loss)
{
    size_t mk = (size_t)M * K, kn = (size_t)K * N, mn = (size_t)M * N;
    uint16_t *Xs = malloc(mk * 2), *Ws = malloc(kn * 2), *Wq = malloc(kn * 2);
    uint16_t *S = malloc((size_t)(K / G) * N * 2), *Yh16 = malloc(mn * 2), *Yr16 = malloc(mn * 2);
    uint8_t *codes = malloc(kn), *zeros = malloc((size_t)(K / G) * N);
    double *Yr = malloc(mn * 8), *Yh = malloc(mn * 8);
    int ok = Xs && Ws && Wq && S && Yh16 && Yr16 && codes && zeros && Yr && Yh;
    if (ok) {
        oracle_migrate(X, W, M, K, N, c, Xs, Ws);
        oracle_quantize(Ws, K, N, G, symmetric, codes, S, symmetric ? NULL : zeros);
        for (int k = 0; k < K; ++k)
            for (int n = 0; n < N; ++n) {
                int z = symmetric ? 8 : zeros[(size_t)(k / G) * N + n];
                Wq[(size_t)k * N + n] =
                    oracle_dequant_one(codes[(size_t)k * N + n], z, S[(size_t)(k / G) * N + n]);
            }
        oracle_matmul_w(X, W, M, K, N, Yr, Yr16);
        oracle_matmul_w(Xs, Wq, M, K, N, Yh, Yh16);
        double sum = 0.0;
        for (size_t i = 0; i < mn; ++i) {
            double d = Yr[i] - oracle_h2d(Yh16[i]);
            sum += d * d;
        }
        *loss = sum / (double)mn;
    }
    free(Xs); free(Ws); free(Wq); free(S); free(Yh16); free(Yr16);
    free(codes); free(zeros); free(Yr); free(Yh);
    return ok ? 0 : -1;
}

int oracle_scale_search(const uint16_t *X, int M, const uint16_t *W, int K, int N, int G,
                        int symmetric, const double *alphas, int n_alpha, double *losses,
                        double *c_best)
{
    double *xbar = malloc((size_t)K * 8), *wbar = malloc((size_t)K * 8), *c = malloc((size_t)K * 8);
    int best = -1;
    if (xbar && wbar && c) {
        oracle_channel_stats(X, M, W, K, N, G, xbar, wbar);
        for (int i = 0; i < n_alpha; ++i) {
            oracle_scale_candidate(xbar, wbar, K, alphas[i], c);
            if (oracle_scale_loss(X, W, M, K, N, G, symmetric, c, &losses[i]) != 0) {
                best = -1;
                break;
            }
            if (best < 0 || losses[i] < losses[best]) best = i;
        }
        if (best >= 0 && c_best) oracle_scale_candidate(xbar, wbar, K, alphas[best], c_best);
    }
    free(xbar); free(wbar); free(c);
    return best;
}
