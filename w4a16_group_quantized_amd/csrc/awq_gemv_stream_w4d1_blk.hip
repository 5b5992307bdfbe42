// Decode GEMV, X staged before the loop: 64-column strips, one segment in flight per wave;
// kernel-private blocked words.
#include "awq_gemv_kernels.h"

namespace awq {
namespace gemv {

hipError_t stream_m_w4_d1_blk(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                              const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                              hipStream_t s) {
    return launch_stream_m<4, 8, 16, 1, 2>(x, qw, sc, qz, y, M, K, N, G, s);
}

}  // namespace gemv
}  // namespace awq
