// Fused W4A16 dequantize-and-multiply for small batches (1 <= M <= 16): the
// decode-time matrix-vector product of AWQ's WQLinear_GEMV module (pyshine.com
// AutoAWQ tour, overview bullets; unfragile.ai AutoAWQ page, the WQLinear
// paragraph: INT4 weights dequantized on the fly, fp16 weights never written).
//
// Bound: HBM.  Every packed weight byte is read exactly once per call, in
// 16-byte coalesced loads; scales and zero points once per group; X and Y are
// small.  Work per packed word must stay below ~20 vector ALU lane-ops for the
// vector units to keep up with 8 TB/s, so the kernel avoids converting codes to
// weights one by one:
//
//  * nibbles become fp16 (1024 + q) with one AND-OR per two codes;
//  * the multiply runs on the matrix cores (v_mfma_f32_16x16x32_f16): one
//    packed word is exactly one lane's B operand (8 k of one column), and the
//    rows of X (up to 16) fill the A operand, so M = 1 and M = 16 cost the same
//    ALU work per weight;
//  * a fifth MFMA against an all-ones B gives sum_k x over the same k, so a
//    segment of L k (L divides G) yields
//        C = sum_k x (1024 + q),  Csum = sum_k x
//    and the segment's contribution is s * (C - (1024 + z) * Csum), i.e.
//    s * sum_k x (q - z), applied once per segment with two FMAs per output.
//    Group sizes that are not a multiple of 32 take the exact path instead:
//    each word is dequantized to fp16 bit-exactly and multiplied directly.
//
// Tiling: one workgroup owns TN = 16 * WPL output columns and all of K.  Each
// lane loads WPL consecutive words (columns) of one packed row; lanes 16j..16j+15
// take packed row 4t + j of step t, so one step covers 32 k.  The NW waves of
// the workgroup take interleaved segments of K; their fp32 partial sums are
// added in LDS in a fixed order (deterministic) and written as fp16.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {
namespace {

template <int WPL>
struct Words {
    uint32_t w[WPL];
};

template <int WPL>
__device__ __forceinline__ Words<WPL> load_words(const uint32_t *p) {
    Words<WPL> r;
    if constexpr (WPL == 1) {
        r.w[0] = p[0];
    } else if constexpr (WPL == 2) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        r.w[0] = v.x;
        r.w[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < WPL / 4; ++i) {
            const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
            r.w[4 * i + 0] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    }
    return r;
}

// WPL consecutive fp16 scales as floats.
template <int WPL>
__device__ __forceinline__ void load_scales(const uint16_t *p, float s[WPL]) {
#pragma unroll
    for (int i = 0; i < WPL; ++i) s[i] = (float)as_half(p[i]);
}

__device__ __forceinline__ half8_t mfma_b(const uint32_t p[4]) {
    return as_half8(make_uint4(p[0], p[1], p[2], p[3]));
}

template <int WPL, int NW, bool FOLD>
__global__ void __launch_bounds__(NW * 64)
gemv_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ Q,
            const uint16_t *__restrict__ S, const uint32_t *__restrict__ QZ,
            uint16_t *__restrict__ Y, int M, int K, int N, int G, int seg_rows) {
    constexpr int TN = 16 * WPL;
    extern __shared__ float red[];  // [NW][M][TN]

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c16 = lane & 15;   // column block (B) / row of X (A) / column of C
    const int kb = lane >> 4;    // which of the 4 packed rows of a step
    const int n0 = blockIdx.x * TN;
    const int ncol = n0 + WPL * c16;
    const bool col_ok = ncol < N;
    const bool row_ok = c16 < M;
    const int KR = K / 8;

    const uint32_t *Qc = Q + ncol;
    const uint16_t *Xr = X + (size_t)c16 * K;

    float acc[WPL][4];
#pragma unroll
    for (int i = 0; i < WPL; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][v] = 0.f;

    if constexpr (FOLD) {
        const half8_t ones = as_half8(make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
        const int nseg = KR / seg_rows;
        for (int seg = wave; seg < nseg; seg += NW) {
            const int r0 = seg * seg_rows;
            const int g = (8 * r0) / G;
            float s[WPL], bz[WPL];
            if (col_ok) {
                load_scales<WPL>(S + (size_t)g * N + ncol, s);
                const uint32_t zw = QZ ? QZ[(size_t)g * (N / 8) + ncol / 8] >> (4 * (ncol % 8))
                                       : 0x88888888u;
#pragma unroll
                for (int i = 0; i < WPL; ++i) bz[i] = 1024.f + (float)((zw >> (4 * i)) & 0xFu);
            } else {
#pragma unroll
                for (int i = 0; i < WPL; ++i) s[i] = bz[i] = 0.f;
            }
            float4_t C[WPL];
#pragma unroll
            for (int i = 0; i < WPL; ++i) C[i] = float4_t{0.f, 0.f, 0.f, 0.f};
            float4_t Cs = {0.f, 0.f, 0.f, 0.f};
            for (int st = 0; st < seg_rows; st += 4) {
                const int r = r0 + st + kb;
                Words<WPL> q;
                if (col_ok) q = load_words<WPL>(Qc + (size_t)r * N);
                else
#pragma unroll
                    for (int i = 0; i < WPL; ++i) q.w[i] = 0u;
                uint4 xa = make_uint4(0u, 0u, 0u, 0u);
                if (row_ok) xa = *reinterpret_cast<const uint4 *>(Xr + 8 * r);
                const half8_t a = as_half8(natural_to_pairs(xa));
#pragma unroll
                for (int i = 0; i < WPL; ++i) {
                    uint32_t p[4];
                    unpack_biased(q.w[i], p);
                    C[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, mfma_b(p), C[i], 0, 0, 0);
                }
                Cs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, Cs, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < WPL; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[i][v] = __builtin_fmaf(s[i], __builtin_fmaf(-bz[i], Cs[v], C[i][v]), acc[i][v]);
        }
    } else {
        // Exact path: each word dequantized bit-exactly, then multiplied.
        float4_t C[WPL];
#pragma unroll
        for (int i = 0; i < WPL; ++i) C[i] = float4_t{0.f, 0.f, 0.f, 0.f};
        const int nstep = (KR + 3) / 4;
        for (int st = wave; st < nstep; st += NW) {
            const int r = 4 * st + kb;
            const bool r_ok = r < KR;
            uint4 xa = make_uint4(0u, 0u, 0u, 0u);
            if (row_ok && r_ok) xa = *reinterpret_cast<const uint4 *>(Xr + 8 * r);
            const half8_t a = as_half8(natural_to_pairs(xa));
            uint32_t d[WPL][4];
            if (col_ok && r_ok) {
                const Words<WPL> q = load_words<WPL>(Qc + (size_t)r * N);
                const int g = (8 * r) / G;
                const uint32_t zw = QZ ? QZ[(size_t)g * (N / 8) + ncol / 8] >> (4 * (ncol % 8))
                                       : 0x88888888u;
                const uint16_t *sp = S + (size_t)g * N + ncol;
#pragma unroll
                for (int i = 0; i < WPL; ++i) {
                    const half_t bz = biased_zero(zw >> (4 * i));
                    const half_t sv = as_half(sp[i]);
                    const half2_t bz2 = {bz, bz}, s2 = {sv, sv};
                    uint32_t p[4];
                    unpack_biased(q.w[i], p);
#pragma unroll
                    for (int j = 0; j < 4; ++j) d[i][j] = dequant_pair(p[j], bz2, s2);
                }
            } else {
#pragma unroll
                for (int i = 0; i < WPL; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) d[i][j] = 0u;
            }
#pragma unroll
            for (int i = 0; i < WPL; ++i)
                C[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, mfma_b(d[i]), C[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < WPL; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][v] = C[i][v];
    }

    // C layout of the 16x16 MFMA: lane (kb, c16) holds rows 4*kb + v, column c16.
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * kb + v;
        if (m < M)
#pragma unroll
            for (int i = 0; i < WPL; ++i) red[(wave * M + m) * TN + WPL * c16 + i] = acc[i][v];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * TN; idx += NW * 64) {
        const int m = idx / TN;
        const int c = idx % TN;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[(w * M + m) * TN + c];
        if (n0 + c < N) Y[(size_t)m * N + n0 + c] = as_u16((half_t)sum);
    }
}

template <int WPL, int NW, bool FOLD>
hipError_t launch(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                  uint16_t *y, int M, int K, int N, int G, int seg_rows, hipStream_t s) {
    constexpr int TN = 16 * WPL;
    const dim3 grid((N + TN - 1) / TN);
    const size_t lds = (size_t)NW * M * TN * sizeof(float);
    hipLaunchKernelGGL((gemv_kernel<WPL, NW, FOLD>), grid, dim3(NW * 64), lds, s, x,
                       reinterpret_cast<const uint32_t *>(qw), sc,
                       reinterpret_cast<const uint32_t *>(qz), y, M, K, N, G, seg_rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                       const int32_t *qzeros, uint16_t *y, int M, int K, int N, int G,
                       hipStream_t s) {
    // Segment length (in packed rows of 8 k) must divide G / 8 and be a whole
    // number of 32-k steps.
    int seg_rows = 0;
    if (G % 128 == 0) seg_rows = 16;
    else if (G % 64 == 0) seg_rows = 8;
    else if (G % 32 == 0) seg_rows = 4;
    if (seg_rows) return launch<4, 8, true>(x, qweight, scales, qzeros, y, M, K, N, G, seg_rows, s);
    return launch<4, 8, false>(x, qweight, scales, qzeros, y, M, K, N, G, 0, s);
}

}  // namespace awq
