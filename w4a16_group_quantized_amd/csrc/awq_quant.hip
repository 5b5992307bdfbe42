// Group quantizer: fp16 W[K][N] -> packed 4-bit codes, fp16 scales and packed
// zero points, the step that produces the layer the fused kernels read.  Each
// group of G weights of a column is rounded to integer levels against a scale
// and zero point (pyshine.com AutoAWQ tour, "The Quantization Flow Up Close":
// the pseudo-quantization pass; "From Install to Your First Model":
// zero_point, q_group_size, w_bit).  The pages give no formula; this is
// textbook min-max, every decision that yields an integer taken in fp32 with
// round-to-nearest-even (correctly rounded division, rint):
//   asymmetric: r = hi - lo (|hi| for a constant group), s = fp16(r / 15),
//               z = clamp(rint(-lo / s), 0, 15)
//   symmetric:  s = fp16(max|w| / 7), z = 8
//   both:       s = 1 if it rounds to 0; q = clamp(rint(w / s) + z, 0, 15)
//
// One thread owns eight consecutive columns of one group: a first pass over the
// group's rows (16-byte loads, coalesced along N) finds the extremes, a second
// pass (re-reading the rows, mostly from cache) computes the codes and writes
// eight packed words per packed row as two 16-byte stores.  Bound: HBM, about
// 2 K N bytes read twice at most, K N / 2 written.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {
namespace {

__device__ __forceinline__ float clamp_code(float v) { return fminf(fmaxf(v, 0.0f), 15.0f); }

__device__ __forceinline__ void load8(const uint16_t *p, float w[8]) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[2 * i] = (float)as_half((uint16_t)u[i]);
        w[2 * i + 1] = (float)as_half((uint16_t)(u[i] >> 16));
    }
}

template <bool SYM>
__global__ void __launch_bounds__(256)
quantize_kernel(const uint16_t *__restrict__ W, uint32_t *__restrict__ Q, uint16_t *__restrict__ S,
                uint32_t *__restrict__ QZ, int K, int N, int G) {
    const int n8 = N / 8;
    const long long total = (long long)(K / G) * n8;
    for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const int g = (int)(t / n8);
        const int n = (int)(t % n8) * 8;
        const uint16_t *wg = W + (size_t)g * G * N + n;

        float lo[8], hi[8], amax[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            lo[i] = __builtin_huge_valf();
            hi[i] = -__builtin_huge_valf();
            amax[i] = 0.0f;
        }
        for (int k = 0; k < G; ++k) {
            float w[8];
            load8(wg + (size_t)k * N, w);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                lo[i] = fminf(lo[i], w[i]);
                hi[i] = fmaxf(hi[i], w[i]);
                amax[i] = fmaxf(amax[i], fabsf(w[i]));
            }
        }
        float sv[8], zv[8];
        uint32_t sh[4] = {0u, 0u, 0u, 0u}, zword = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float r;
            if (SYM) {
                r = amax[i] / 7.0f;
            } else {
                float range = hi[i] - lo[i];
                if (range == 0.0f) range = fabsf(hi[i]);
                r = range / 15.0f;
            }
            uint16_t s16 = as_u16((half_t)r);
            if ((s16 & 0x7FFFu) == 0u) s16 = 0x3C00u;   // 1.0
            sv[i] = (float)as_half(s16);
            zv[i] = SYM ? 8.0f : clamp_code(__builtin_rintf(-lo[i] / sv[i]));
            sh[i / 2] |= (uint32_t)s16 << (16 * (i % 2));
            zword |= (uint32_t)zv[i] << (4 * i);
        }
        *reinterpret_cast<uint4 *>(S + (size_t)g * N + n) = make_uint4(sh[0], sh[1], sh[2], sh[3]);
        if (!SYM) QZ[(size_t)g * n8 + n / 8] = zword;

        for (int r = 0; r < G / 8; ++r) {
            uint32_t word[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float w[8];
                load8(wg + (size_t)(8 * r + j) * N, w);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    word[i] |= (uint32_t)clamp_code(__builtin_rintf(w[i] / sv[i]) + zv[i]) << (4 * j);
            }
            uint32_t *qrow = Q + (size_t)(g * (G / 8) + r) * N + n;
            reinterpret_cast<uint4 *>(qrow)[0] = make_uint4(word[0], word[1], word[2], word[3]);
            reinterpret_cast<uint4 *>(qrow)[1] = make_uint4(word[4], word[5], word[6], word[7]);
        }
    }
}

}  // namespace

hipError_t launch_quantize(const uint16_t *w, int32_t *qweight, uint16_t *scales, int32_t *qzeros,
                           int K, int N, int G, bool symmetric, hipStream_t s) {
    const long long threads = (long long)(K / G) * (N / 8);
    long long blocks = (threads + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    auto *q = reinterpret_cast<uint32_t *>(qweight);
    auto *z = reinterpret_cast<uint32_t *>(qzeros);
    if (symmetric)
        hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, w, q, scales,
                           z, K, N, G);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, w, q,
                           scales, z, K, N, G);
    return hipGetLastError();
}

}  // namespace awq
