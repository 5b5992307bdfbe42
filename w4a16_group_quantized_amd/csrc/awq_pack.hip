// Packing and exact dequantization kernels.
//
// Packing puts eight 4-bit weights into one 32-bit word, as AWQ stores its
// qweight (mbrenndoerfer.com, "AWQ > Implementation", "Understanding the
// Quantization Structure"); both run once per layer, when it is loaded.  The
// dequantization kernel writes w = fp16_rne(s * (q - z)) (fak explainer,
// "Dequantization Formula", for the symmetric zero 8) and exposes the exact
// weights the fused kernels compute in registers.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {
namespace {

// One thread per four consecutive columns of one packed row: eight 4-byte code
// loads (one per k), four words out as one 16-byte store.
__global__ void __launch_bounds__(256)
pack_kernel(const uint8_t *__restrict__ codes, int32_t *__restrict__ qweight, int K, int N) {
    const int n4 = N / 4;
    const long long total = (long long)(K / 8) * n4;
    for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const int r = (int)(t / n4);
        const int n = (int)(t % n4) * 4;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t c = *reinterpret_cast<const uint32_t *>(
                codes + (size_t)(8 * r + j) * N + n);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] |= ((c >> (8 * i)) & 0xFu) << (4 * j);
        }
        *reinterpret_cast<uint4 *>(qweight + (size_t)r * N + n) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// One thread per output word: eight consecutive zero points of one group.
__global__ void __launch_bounds__(256)
pack_zeros_kernel(const uint8_t *__restrict__ zeros, int32_t *__restrict__ qzeros, int groups,
                  int N) {
    const int n8 = N / 8;
    const long long total = (long long)groups * n8;
    for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const uint2 z = *reinterpret_cast<const uint2 *>(zeros + t * 8);
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w |= ((z.x >> (8 * j)) & 0xFu) << (4 * j);
            w |= ((z.y >> (8 * j)) & 0xFu) << (4 * (j + 4));
        }
        qzeros[t] = (int32_t)w;
    }
}

// One thread per four consecutive words of one packed row: 4 columns x 8 k.
__global__ void __launch_bounds__(256)
dequant_kernel(const uint32_t *__restrict__ qweight, const uint16_t *__restrict__ scales,
               const uint32_t *__restrict__ qzeros, uint16_t *__restrict__ w, int K, int N,
               int G, int il) {
    const int n4 = N / 4;
    const long long total = (long long)(K / 8) * n4;
    const uint32_t nmask = nibble_mask_vgpr();
    for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const int r = (int)(t / n4);
        const int n = (int)(t % n4) * 4;
        const int g = (8 * r) / G;
        const bool blk = il == 2;   // il: the qweight layout (nonzero: interleaved nibbles)
        const uint4 q = *reinterpret_cast<const uint4 *>(qweight + (size_t)r * q_pitch(blk, N) +
                                                          q_col(blk, n, K / 8));
        const uint2 s = *reinterpret_cast<const uint2 *>(scales + (size_t)g * N + n);
        const uint32_t zw = qzeros ? qzeros[(size_t)g * (N / 8) + n / 8] >> (4 * (n % 8))
                                   : 0x8888u;
        uint32_t qs[4] = {q.x, q.y, q.z, q.w};
        if (il)   // interleaved words: back to the canonical nibble order first
#pragma unroll
            for (int i = 0; i < 4; ++i) qs[i] = deinterleave_word(qs[i]);
        const uint16_t ss[4] = {(uint16_t)s.x, (uint16_t)(s.x >> 16), (uint16_t)s.y,
                                (uint16_t)(s.y >> 16)};
        uint4 col[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            col[i] = dequant_word_natural(qs[i], nmask, biased_zero(zw >> (4 * i)), as_half(ss[i]));
        // col[i] holds k = 8r..8r+7 of column n+i; write row by row, 4 columns at a time.
        const uint32_t *c = reinterpret_cast<const uint32_t *>(col);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = (c[4 * i + j / 2] >> (16 * (j % 2))) & 0xFFFFu;
            *reinterpret_cast<uint2 *>(w + (size_t)(8 * r + j) * N + n) =
                make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
    }
}

unsigned grid_for(long long threads) {
    long long blocks = (threads + 255) / 256;
    // enough blocks to fill 256 CUs many times over; the kernels loop beyond it
    return (unsigned)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_pack(const uint8_t *codes, int32_t *qweight, int K, int N, hipStream_t s) {
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for((long long)(K / 8) * (N / 4))), dim3(256), 0, s,
                       codes, qweight, K, N);
    return hipGetLastError();
}

hipError_t launch_pack_zeros(const uint8_t *zeros, int32_t *qzeros, int groups, int N,
                             hipStream_t s) {
    hipLaunchKernelGGL(pack_zeros_kernel, dim3(grid_for((long long)groups * (N / 8))), dim3(256),
                       0, s, zeros, qzeros, groups, N);
    return hipGetLastError();
}

hipError_t launch_dequant(const int32_t *qweight, const uint16_t *scales, const int32_t *qzeros,
                          uint16_t *w, int K, int N, int G, int il, hipStream_t s) {
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for((long long)(K / 8) * (N / 4))), dim3(256), 0,
                       s, reinterpret_cast<const uint32_t *>(qweight), scales,
                       reinterpret_cast<const uint32_t *>(qzeros), w, K, N, G, il);
    return hipGetLastError();
}

// Packed words from one layout to another: four words (packed row r, columns
// n .. n + 3) per thread, read where layout `from` keeps them and written where
// `to` does (q_col, q_pitch: the blocked layout moves words, the others keep
// them in place), each word's nibbles permuted between the canonical and the
// interleaved order when the two differ (interleave_word: a byte swap and a
// nibble swap).  With src == dst the positions must agree (the caller checks),
// and each thread then reads and writes only its own four words.
__global__ void __launch_bounds__(256)
repack_kernel(const uint32_t *src, uint32_t *dst, int K, int N, int from, int to) {
    const int n4 = N / 4, KR = K / 8;
    const long long total = (long long)KR * n4;
    const bool fblk = from == 2, tblk = to == 2;
    const int nib = (to != 0) - (from != 0);   // +1 interleave, -1 back to canonical, 0 keep
    for (long long t = blockIdx.x * 256LL + threadIdx.x; t < total; t += (long long)gridDim.x * 256) {
        const int r = (int)(t / n4);
        const int n = (int)(t % n4) * 4;
        uint4 v = *reinterpret_cast<const uint4 *>(src + (size_t)r * q_pitch(fblk, N) +
                                                   q_col(fblk, n, KR));
        if (nib > 0) {
            v.x = interleave_word(v.x);
            v.y = interleave_word(v.y);
            v.z = interleave_word(v.z);
            v.w = interleave_word(v.w);
        } else if (nib < 0) {
            v.x = deinterleave_word(v.x);
            v.y = deinterleave_word(v.y);
            v.z = deinterleave_word(v.z);
            v.w = deinterleave_word(v.w);
        }
        *reinterpret_cast<uint4 *>(dst + (size_t)r * q_pitch(tblk, N) + q_col(tblk, n, KR)) = v;
    }
}

hipError_t launch_repack(const int32_t *src, int32_t *dst, int K, int N, int from, int to,
                         hipStream_t s) {
    hipLaunchKernelGGL(repack_kernel, dim3(grid_for((long long)(K / 8) * (N / 4))), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t *>(src), reinterpret_cast<uint32_t *>(dst),
                       K, N, from, to);
    return hipGetLastError();
}

}  // namespace awq
