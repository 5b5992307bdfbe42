// Small-batch GEMV, X staged segment by segment: 64-column strips; kernel-private blocked
// words.
#include "awq_gemv_kernels.h"

namespace awq {
namespace gemv {

hipError_t prog_w4_blk(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                       const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                       hipStream_t s) {
    return launch_stream_prog<4, 8, 1, false, 2>(x, qw, sc, qz, y, M, K, N, G, s);
}

}  // namespace gemv
}  // namespace awq
