// Small-batch GEMV, X staged segment by segment: 128 columns per workgroup (a 64-column
// strip of each half of the layer where N is a multiple of 16, else one strip); canonical words.
#include "awq_gemv_kernels.h"

namespace awq {
namespace gemv {

hipError_t prog_w8(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                   const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                   hipStream_t s) {
    // A strip of each half of the columns per workgroup (N a multiple of 16).
    if (N % 16 == 0) return launch_stream_prog<8, 8, 1, 2, false>(x, qw, sc, qz, y, M, K, N, G, s);
    return launch_stream_prog<8, 8, 1, 0, false>(x, qw, sc, qz, y, M, K, N, G, s);
}

}  // namespace gemv
}  // namespace awq
