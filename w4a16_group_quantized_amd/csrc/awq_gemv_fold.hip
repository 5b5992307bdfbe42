// GEMV for shapes outside the staged kernel: the folded kernel (G a multiple of 32) and the exact
// one.
#include "awq_gemv_kernels.h"

namespace awq {
namespace gemv {

hipError_t fold_w2_s16(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                       const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                       hipStream_t s) {
    return launch_fold_any<2, 16>(x, qw, sc, qz, y, M, K, N, G, il, s);
}

hipError_t fold_w4_s16(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                       const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                       hipStream_t s) {
    return launch_fold_any<4, 16>(x, qw, sc, qz, y, M, K, N, G, il, s);
}

hipError_t fold_w4_s8(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                      const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                      hipStream_t s) {
    return launch_fold_any<4, 8>(x, qw, sc, qz, y, M, K, N, G, il, s);
}

hipError_t fold_w4_s4(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                      const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                      hipStream_t s) {
    return launch_fold_any<4, 4>(x, qw, sc, qz, y, M, K, N, G, il, s);
}

hipError_t exact_w4(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                    const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                    hipStream_t s) {
    return launch_exact<4, 8>(x, qw, sc, qz, y, M, K, N, G, il, s);
}

}  // namespace gemv
}  // namespace awq
