/*
 * Plain CPU oracle for the W4A16 group-quantized linear layer.
 * TEST INFRASTRUCTURE ONLY: never included by, linked into or called from the
 * HIP library.  See oracle.c for what each function computes and the passages
 * of the AWQ pages it follows.
 *
 * Layouts (all row-major, fp16 given as IEEE binary16 bit patterns):
 *   codes  uint8 [K][N]       4-bit codes 0..15 (higher bits ignored)
 *   Q      int32 [K/8][N]     code of (k, n) in bits 4*(k%8).. of Q[k/8][n]
 *   zeros  uint8 [K/G][N]     4-bit zero points
 *   QZ     int32 [K/G][N/8]   zero of (g, n) in bits 4*(n%8).. of QZ[g][n/8];
 *                             NULL means the symmetric zero point 8
 *   S      fp16  [K/G][N]     one scale per group and column
 *   X      fp16  [M][K]       activations
 *   W      fp16  [K][N]       dequantized weight
 *   Y64    fp64  [M][N]       exact-order fp64 sum; Y16 its fp16 rounding
 *   H16    fp16  [M][N/2]     fused gate/up output, columns [gate | up] of Y
 *   xbar, wbar, c  fp64 [K]   per-input-channel statistics and scales
 */
#ifndef W4A16_ORACLE_H
#define W4A16_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double   oracle_h2d(uint16_t h);
uint16_t oracle_d2h(double x);
void     oracle_h2d_n(const uint16_t *h, size_t count, double *out);
void     oracle_d2h_n(const double *x, size_t count, uint16_t *out);

void oracle_pack(const uint8_t *codes, int K, int N, int32_t *Q);
void oracle_pack_zeros(const uint8_t *zeros, int groups, int N, int32_t *QZ);
int  oracle_code(const int32_t *Q, int N, int k, int n);
int  oracle_zero(const int32_t *QZ, int N, int g, int n);
void oracle_unpack(const int32_t *Q, int K, int N, uint8_t *codes);
void oracle_unpack_zeros(const int32_t *QZ, int groups, int N, uint8_t *zeros);
/* Kernel-private layout: nibble of k % 8 = j moved to 4 (j % 2) + j / 2. */
void oracle_interleave(const int32_t *Q, int K, int N, int32_t *out);
void oracle_deinterleave(const int32_t *Q, int K, int N, int32_t *out);
void oracle_block(const int32_t *Q, int K, int N, int32_t *out);
void oracle_unblock(const int32_t *B, int K, int N, int32_t *out);

uint16_t oracle_dequant_one(int q, int z, uint16_t s);
void oracle_dequant(const int32_t *Q, const uint16_t *S, const int32_t *QZ,
                    int K, int N, int G, uint16_t *W);

void oracle_matmul_w(const uint16_t *X, const uint16_t *W, int M, int K, int N,
                     double *Y64, uint16_t *Y16);
int  oracle_linear(const uint16_t *X, const int32_t *Q, const uint16_t *S,
                   const int32_t *QZ, int M, int K, int N, int G,
                   double *Y64, uint16_t *Y16);

void   oracle_quantize(const uint16_t *W, int K, int N, int G, int symmetric,
                       uint8_t *codes, uint16_t *S, uint8_t *zeros);
double oracle_silu(double t);
void   oracle_gate_up(const double *Y64, int M, int I, uint16_t *H16);

void oracle_channel_stats(const uint16_t *X, int M, const uint16_t *W, int K, int N, int G,
                          double *xbar, double *wbar);
void oracle_scale_candidate(const double *xbar, const double *wbar, int K, double alpha, double *c);
void oracle_migrate(const uint16_t *X, const uint16_t *W, int M, int K, int N, const double *c,
                    uint16_t *Xs, uint16_t *Ws);
int  oracle_scale_loss(const uint16_t *X, const uint16_t *W, int M, int K, int N, int G,
                       int symmetric, const double *c, double *loss);
int  oracle_scale_search(const uint16_t *X, int M, const uint16_t *W, int K, int N, int G,
                         int symmetric, const double *alphas, int n_alpha, double *losses,
                         double *c_best);

#ifdef __cplusplus
}
#endif

#endif
