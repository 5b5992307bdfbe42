// Entry points of the batch GEMM (AWQ's WQLinear_GEMM module, "GEMM for batch
// inference": unfragile.ai AutoAWQ page, the WQLinear paragraph), the general
// kernel's launcher and the split-K reduction.  The kernels and their design
// are in awq_gemm_kernels.h; awq_gemm_canon.hip and awq_gemm_il.hip
// instantiate them for the two word layouts.
#include "awq_gemm_kernels.h"

namespace awq {
namespace gemm {

template <int BM, bool SYM>
hipError_t launch_general_bm(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                          const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                          hipStream_t s) {
    const long long tiles = (long long)((M + BM - 1) / BM) * ((N + kBN - 1) / kBN);
    hipLaunchKernelGGL((gemm_kernel<BM, SYM>), dim3((unsigned)tiles), dim3(256), 0, s, x,
                       reinterpret_cast<const uint32_t *>(qw), sc,
                       reinterpret_cast<const uint32_t *>(qz), y, M, K, N, G, il);
    return hipGetLastError();
}

hipError_t launch_general(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                          const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                          hipStream_t s) {
    return qz == nullptr ? launch_general_bm<128, true>(x, qw, sc, qz, y, M, K, N, G, il, s)
                         : launch_general_bm<128, false>(x, qw, sc, qz, y, M, K, N, G, il, s);
}

// Y = fp16(sum over the slices of part[s]), slices added in order.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float *__restrict__ part, int splits, long long count,
                     uint16_t *__restrict__ Y) {
    const long long quads = count / 4;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < quads; i += (long long)gridDim.x * 256) {
        float4 a = reinterpret_cast<const float4 *>(part)[i];
        for (int sl = 1; sl < splits; ++sl) {
            const float4 b = reinterpret_cast<const float4 *>(part + (size_t)sl * count)[i];
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        reinterpret_cast<uint2 *>(Y)[i] =
            make_uint2((uint32_t)as_u16((half_t)a.x) | ((uint32_t)as_u16((half_t)a.y) << 16),
                       (uint32_t)as_u16((half_t)a.z) | ((uint32_t)as_u16((half_t)a.w) << 16));
    }
}

}  // namespace gemm

bool gemm_splitk_supported(int K, int G, int splits) { return gemm::splitk_bk(K, G, splits) != 0; }

size_t gemm_splitk_workspace(int M, int N, int splits) {
    return (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_gemm_splitk(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                              const int32_t *qzeros, uint16_t *y, int M, int K, int N, int G,
                              int splits, void *workspace, int il, hipStream_t s) {
    auto *part = static_cast<float *>(workspace);
    auto *split = il == 2 ? gemm::split_blk : il ? gemm::split_il : gemm::split_canon;
    const hipError_t e = split(x, qweight, scales, qzeros, part, M, K, N, G, splits, s);
    if (e != hipSuccess) return e;
    const long long count = (long long)M * N;
    long long blocks = (count / 4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(gemm::splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part,
                       splits, count, y);
    return hipGetLastError();
}

bool gemm_gate_up_supported(int K, int N, int G) {
    return N % 16 == 0 && G % gemm::kBK == 0 && K % (gemm::kRing * gemm::kBK) == 0;
}

hipError_t launch_gemm_gate_up(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                               const int32_t *qzeros, uint16_t *h, int M, int K, int N, int G,
                               int il, hipStream_t s) {
    auto *gate_up = il == 2 ? gemm::gate_up_blk : il ? gemm::gate_up_il : gemm::gate_up_canon;
    return gate_up(x, qweight, scales, qzeros, h, M, K, N, G, s);
}

hipError_t launch_gemm(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                       const int32_t *qzeros, uint16_t *y, int M, int K, int N, int G, int il,
                       hipStream_t s) {
    auto *plain = il == 2 ? gemm::plain_blk : il ? gemm::plain_il : gemm::plain_canon;
    return plain(x, qweight, scales, qzeros, y, M, K, N, G, s);
}

}  // namespace awq

