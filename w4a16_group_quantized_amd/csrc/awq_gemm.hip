// Fused W4A16 dequantize-and-multiply for batches: AWQ's WQLinear_GEMM module,
// "GEMM for batch inference" (unfragile.ai AutoAWQ page, the WQLinear
// paragraph; pyshine.com AutoAWQ tour, overview bullets).  At M in the
// thousands this is a dense contraction, bound by the matrix cores.
//
// Per workgroup (256 threads, four waves in a 2 x 2 grid): a BM x BN tile of Y,
// K walked in BK steps.  Each step
//   * loads the BM x BK slice of X (16-byte loads) and the BK/8 x BN packed
//     words of the weight, one 16-byte load (four columns) per thread;
//   * dequantizes the words bit-exactly (w = fp16_rne(s (q - z))) and stores
//     them in LDS column-major (eight consecutive k of one column = 16 bytes),
//     which is the B operand layout of v_mfma_f32_32x32x16_f16;
//   * runs the wave's (BM/2) x (BN/2) sub-tile of MFMAs with fp32 accumulators.
// The next step's global loads are issued before the current step's MFMAs and
// land in the other half of a double-buffered LDS.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {
namespace {

template <int BM, int BN, int BK>
__global__ void __launch_bounds__(256)
gemm_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ Q,
            const uint16_t *__restrict__ S, const uint32_t *__restrict__ QZ,
            uint16_t *__restrict__ Y, int M, int K, int N, int G) {
    constexpr int LDA = BK + 8;  // halves per LDS row (16-byte pad against bank conflicts)
    constexpr int LDB = BK + 8;
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int ACH = BM * BK / 8 / 256;         // 16-byte X chunks per thread per step
    constexpr int BCH = (BK / 8) * (BN / 4) / 256; // 4-word packed chunks per thread per step
    static_assert(ACH >= 1 && BCH >= 1, "tile too small for 256 threads");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDA];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = (N + BN - 1) / BN;
    const int m0 = (int)(blockIdx.x / tiles_n) * BM;
    const int n0 = (int)(blockIdx.x % tiles_n) * BN;
    const int KR = K / 8;
    const int KT = (K + BK - 1) / BK;
    const uint32_t nmask = nibble_mask_vgpr();

    uint4 a_reg[ACH];
    uint4 q_reg[BCH];
    uint2 s_reg[BCH];
    uint32_t z_reg[BCH];
    bool b_ok[BCH];

    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int c = tid + 256 * i;
            const int row = c / (BK / 8);
            const int gk = kt * BK + (c % (BK / 8)) * 8;
            const int gm = m0 + row;
            a_reg[i] = (gm < M && gk < K)
                           ? *reinterpret_cast<const uint4 *>(X + (size_t)gm * K + gk)
                           : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int c = tid + 256 * i;
            const int r = kt * (BK / 8) + c / (BN / 4);
            const int n = n0 + (c % (BN / 4)) * 4;
            b_ok[i] = r < KR && n < N;
            if (b_ok[i]) {
                const int g = (8 * r) / G;
                q_reg[i] = *reinterpret_cast<const uint4 *>(Q + (size_t)r * N + n);
                s_reg[i] = *reinterpret_cast<const uint2 *>(S + (size_t)g * N + n);
                z_reg[i] = QZ ? QZ[(size_t)g * (N / 8) + n / 8] >> (4 * (n % 8)) : 0x8888u;
            }
        }
    };

    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int c = tid + 256 * i;
            const int row = c / (BK / 8);
            const int kc = c % (BK / 8);
            *reinterpret_cast<uint4 *>(&As[buf][row * LDA + kc * 8]) = a_reg[i];
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int c = tid + 256 * i;
            const int kq = c / (BN / 4);
            const int nl = (c % (BN / 4)) * 4;
            const uint32_t qs[4] = {q_reg[i].x, q_reg[i].y, q_reg[i].z, q_reg[i].w};
            const uint16_t ss[4] = {(uint16_t)s_reg[i].x, (uint16_t)(s_reg[i].x >> 16),
                                    (uint16_t)s_reg[i].y, (uint16_t)(s_reg[i].y >> 16)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 w = b_ok[i] ? dequant_word_natural(qs[j], nmask, biased_zero(z_reg[i] >> (4 * j)),
                                                               as_half(ss[j]))
                                        : make_uint4(0u, 0u, 0u, 0u);
                *reinterpret_cast<uint4 *>(&Bs[buf][(nl + j) * LDB + kq * 8]) = w;
            }
        }
    };

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    gload(0);
    sstore(0);
    __syncthreads();

    const int lrow = lane & 31;
    const int lk = 8 * (lane >> 5);
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            half8_t a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = as_half8(*reinterpret_cast<const uint4 *>(
                    &As[buf][(wm * WTM + 32 * i + lrow) * LDA + kk + lk]));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                b[j] = as_half8(*reinterpret_cast<const uint4 *>(
                    &Bs[buf][(wn * WTN + 32 * j + lrow) * LDB + kk + lk]));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore(buf ^ 1);
        __syncthreads();
    }

    // C layout of the 32x32 MFMA: lane l holds column l % 32 and, for register
    // v, row 8 * (v / 4) + 4 * (l / 32) + v % 4.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WTN + 32 * j + lrow;
            if (col >= N) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * WTM + 32 * i + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
                if (row < M) Y[(size_t)row * N + col] = as_u16((half_t)acc[i][j][v]);
            }
        }
}

}  // namespace

hipError_t launch_gemm(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                       const int32_t *qzeros, uint16_t *y, int M, int K, int N, int G,
                       hipStream_t s) {
    constexpr int BM = 128, BN = 128, BK = 64;
    const dim3 grid((unsigned)(((N + BN - 1) / BN) * (long long)((M + BM - 1) / BM)));
    hipLaunchKernelGGL((gemm_kernel<BM, BN, BK>), grid, dim3(256), 0, s, x,
                       reinterpret_cast<const uint32_t *>(qweight), scales,
                       reinterpret_cast<const uint32_t *>(qzeros), y, M, K, N, G);
    return hipGetLastError();
}

}  // namespace awq
