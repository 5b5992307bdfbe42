// Fused gate/up GEMV (h = SiLU(gate) * up) on kernel-private blocked words.
#include "awq_gemv_kernels.h"

namespace awq {
namespace gemv {

hipError_t gate_up_blk(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                       const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                       hipStream_t s) {
    return gate_up_layout<2>(x, qw, sc, qz, y, M, K, N, G, s);
}

}  // namespace gemv
}  // namespace awq
