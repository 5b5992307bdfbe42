// Fused gate/up GEMV (h = SiLU(gate) * up), the staged kernel in its gate/up mode.
#include "awq_gemv_kernels.h"

namespace awq {

bool gemv_gate_up_supported(int M, int K, int N, int G) {
    using namespace gemv;
    if (M < 1 || M > 16 || N % 16 != 0) return false;
    if (stream_fits_prog(M, K, N, G, 8, 8, 1))
        return true;   // X staged segment by segment: any K
    return stream_fits(M, K, N, G, 8, 8, 16, 1) || stream_fits(M, K, N, G, 8, 2, 16, 1) ||
           stream_fits(M, K, N, G, 8, 1, 16, 1);
}

hipError_t launch_gemv_gate_up(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                               const int32_t *qzeros, uint16_t *h, int M, int K, int N, int G,
                               int il, hipStream_t s) {
    auto *gate_up = il == 2 ? gemv::gate_up_blk : il ? gemv::gate_up_il : gemv::gate_up;
    return gate_up(x, qweight, scales, qzeros, h, M, K, N, G, s);
}

}  // namespace awq
