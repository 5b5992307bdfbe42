// Host-side launchers behind the C ABI of include/awq.h.  Arguments reach them
// already validated (shapes, alignment, non-null pointers, M >= 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

hipError_t launch_pack(const uint8_t *codes, int32_t *qweight, int K, int N, hipStream_t s);
hipError_t launch_pack_zeros(const uint8_t *zeros, int32_t *qzeros, int groups, int N,
                             hipStream_t s);
// `il` (every launcher below that reads a layer): the layout of the packed
// words, AWQ_LAYOUT_* (0 canonical; 1 interleaved and 2 blocked, the
// kernel-private ones of awq_repack).
hipError_t launch_dequant(const int32_t *qweight, const uint16_t *scales, const int32_t *qzeros,
                          uint16_t *w, int K, int N, int G, int il, hipStream_t s);
// Packed words [K/8][N] from layout `from` to layout `to` (src may equal dst
// when neither or both layouts are blocked).
hipError_t launch_repack(const int32_t *src, int32_t *dst, int K, int N, int from, int to,
                         hipStream_t s);
hipError_t launch_gemv(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                       const int32_t *qzeros, uint16_t *y, int M, int K, int N, int G, int il,
                       hipStream_t s);
hipError_t launch_quantize(const uint16_t *w, int32_t *qweight, uint16_t *scales, int32_t *qzeros,
                           int K, int N, int G, bool symmetric, hipStream_t s);
// The same for W'(k, n) = fp16(c[k] w(k, n)), formed as the rows are read
// (c: device fp32 [K]); no W' is written.
hipError_t launch_quantize_migrated(const uint16_t *w, const float *c, int32_t *qweight,
                                    uint16_t *scales, int32_t *qzeros, int K, int N, int G,
                                    bool symmetric, hipStream_t s);
// Fused gate/up (layer columns [gate | up], h = fp16(SiLU(gate) * up)).
bool gemv_gate_up_supported(int M, int K, int N, int G);
hipError_t launch_gemv_gate_up(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                               const int32_t *qzeros, uint16_t *h, int M, int K, int N, int G,
                               int il, hipStream_t s);
bool gemm_gate_up_supported(int K, int N, int G);
hipError_t launch_gemm_gate_up(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                               const int32_t *qzeros, uint16_t *h, int M, int K, int N, int G,
                               int il, hipStream_t s);
hipError_t launch_gemm(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                       const int32_t *qzeros, uint16_t *y, int M, int K, int N, int G, int il,
                       hipStream_t s);
// Split K: slices of K / splits summed by separate workgroups into fp32
// partials (workspace: splits * M * N floats), then added in slice order.
bool gemm_splitk_supported(int K, int G, int splits);
size_t gemm_splitk_workspace(int M, int N, int splits);
hipError_t launch_gemm_splitk(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                              const int32_t *qzeros, uint16_t *y, int M, int K, int N, int G,
                              int splits, void *workspace, int il, hipStream_t s);
// The same on the library's static per-device scratch (splits * M * N * 4
// bytes must be at most kStaticScratchBytes; hipErrorInvalidValue otherwise).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t launch_gemm_splitk_static(const uint16_t *x, const int32_t *qweight,
                                     const uint16_t *scales, const int32_t *qzeros, uint16_t *y,
                                     int M, int K, int N, int G, int splits, int il, hipStream_t s);
// Scale search (per-channel statistics, candidates, migrated layer, loss).
constexpr int kScaleSearchMaxAlphas = 64;
size_t channel_stats_workspace(int M, int K, int N, int G);
size_t scale_search_workspace(int M, int K, int N, int G);
hipError_t launch_channel_stats(const uint16_t *x, int M, const uint16_t *w, int K, int N, int G,
                                float *xbar, float *wbar, void *workspace, hipStream_t s);
// alphas: host array of n_alpha values (read during the call).
hipError_t launch_scale_search(const uint16_t *x, int M, const uint16_t *w, int K, int N, int G,
                               bool symmetric, const float *alphas, int n_alpha, double *losses,
                               int32_t *best, float *best_scales, void *workspace, hipStream_t s);

}  // namespace awq
