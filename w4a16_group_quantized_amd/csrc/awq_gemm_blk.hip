// The batch GEMM's 32x32x16 MFMA kernels on kernel-private blocked words: the plain,
// split-K and fused gate/up launchers.
#include "awq_gemm_kernels.h"

namespace awq {
namespace gemm {

hipError_t plain_blk(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                     uint16_t *y, int M, int K, int N, int G, hipStream_t s) {
    return launch_layout<2>(x, qw, sc, qz, y, M, K, N, G, s);
}

hipError_t split_blk(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                     float *part, int M, int K, int N, int G, int splits, hipStream_t s) {
    return split_layout<2>(x, qw, sc, qz, part, M, K, N, G, splits, s);
}

hipError_t gate_up_blk(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                       uint16_t *h, int M, int K, int N, int G, hipStream_t s) {
    return gate_up_layout<2>(x, qw, sc, qz, h, M, K, N, G, s);
}

}  // namespace gemm
}  // namespace awq
