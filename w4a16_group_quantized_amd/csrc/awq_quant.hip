// Group quantizer: fp16 W[K][N] -> packed 4-bit codes, fp16 scales and packed
// zero points, the step that produces the layer the fused kernels read.  Each
// group of G weights of a column is rounded to integer levels against a scale
// and zero point (pyshine.com AutoAWQ tour, "The Quantization Flow Up Close":
// the pseudo-quantization pass; "From Install to Your First Model":
// zero_point, q_group_size, w_bit).  The pages give no formula; this is
// textbook min-max:
//   asymmetric: r = hi - lo (|hi| for a constant group), s = fp16(r / 15),
//               z = clamp(rint(-lo / s), 0, 15)
//   symmetric:  s = fp16(max|w| / 7), z = 8
//   both:       s = 1 if it rounds to 0; q = clamp(rint(w / s) + z, 0, 15)
// The scale is the exact real r / 15 (or r / 7) rounded once to fp16: the
// range of two fp16 values is exact in fp64 (at most 40 significant bits), and
// the fp64 quotient is never closer to an fp16 rounding midpoint than the real
// one unless both equal it (they differ by 2^-53 relative; a real quotient
// that is not a midpoint lies at least 2^-42 relative away from all of them),
// so rounding it to fp16 once gives the exact scale.  The integer decisions (z
// and the codes) are taken in fp32 with round-to-nearest-even (correctly
// rounded division, rint).
//
// A workgroup of WPG waves owns one group of 64 columns: lane (c, r) =
// (lane / 8, lane % 8) of wave v takes the 8 columns 8 c .. 8 c + 7 and the
// rows r + 8 v, + 8 WPG, ... of the group.  A first pass (16-byte loads, 8 in
// flight per lane, 128 contiguous bytes per row across the wave's column
// chunks) finds each column's extremes; shuffles over the eight row lanes of a
// chunk, then LDS across the waves, complete them (exactly, in any order).  A
// second pass takes packed rows p = r + 8 v, + 8 WPG, ...: it re-reads the
// group's rows 8 p .. 8 p + 7 (from cache), computes the codes and writes the
// eight packed words of the chunk as two 16-byte stores.  Bound: HBM, 2 K N
// bytes read, K N / 2 written.  WPG = 4, 8 or 16 for layers with few (group,
// column) tiles and long groups, so that those are read by enough lanes at once.
// Groups of 64 to 256 rows are instead read once: the first pass takes the
// second pass's packed rows and keeps them in registers.
//
// The extremes are taken on the fp16 values themselves (packed min / max,
// exact).  rint(w / s) is decided from w * (1 / s): that product is within
// 2^-22 |w / s| of the true quotient, so unless it lies that close to a
// half-integer its rint equals rint of the correctly rounded quotient; the
// values that close divide exactly.  With fp16 weights and scales exact ties
// (w = (k + 1/2) s) are common, so the test is made per value: redoing a
// whole packed row whenever one of its values is close costs more.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {
namespace {

__device__ __forceinline__ float clamp_code(float v) { return fminf(fmaxf(v, 0.0f), 15.0f); }

__device__ __forceinline__ uint4 load16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// rint(w / s) with the quotient correctly rounded to fp32 first; inv = 1 / s.
__device__ __forceinline__ float rint_quotient(float w, float s, float inv) {
    const float q = w * inv;
    const float t = __builtin_rintf(q);
    if (fabsf(q - t) >= 0.5f - fabsf(q) * 0x1p-21f) return __builtin_rintf(w / s);
    return t;
}

// fp16 bits of a finite x >= 0, rounded once to nearest, ties to even.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
    if (x >= 65520.0) return 0x7C00u;                // rounds to infinity
    if (x == 0.0) return 0u;
    int e = ilogb(x);
    if (e < -14) e = -14;                            // subnormals share exponent -14
    int n = (int)__builtin_rint(ldexp(x, 10 - e));   // exact scaling, then RNE
    if (n == 2048) {                                 // carried into the next binade
        n = 1024;
        ++e;
    }
    return n < 1024 ? (uint16_t)n : (uint16_t)(((e + 15) << 10) | (n - 1024));
}

// Columns of one column chunk, one chunk per eight lanes.
constexpr int kRowLanes = 8;

// HOLD > 0 (one wave, G = 64 HOLD): the first pass already reads the packed
// rows the second pass quantizes, p = r, r + 8, ..., and keeps them in
// registers (HOLD x 8 chunks per lane), so the group is read once.
// MIG: the layer quantized is W'(k, n) = fp16(c[k] w(k, n)) (fp32 product,
// one rounding), formed from each row as it is loaded; c: fp32 [K].
template <bool SYM, int WPG, int HOLD = 0, bool MIG = false>
__global__ void __launch_bounds__(64 * WPG)
quantize_kernel(const uint16_t *__restrict__ W, uint32_t *__restrict__ Q, uint16_t *__restrict__ S,
                uint32_t *__restrict__ QZ, int K, int N, int G, int tiles_n,
                const float *__restrict__ c_rows) {
    constexpr int kStride = kRowLanes * WPG;     // rows between a lane's consecutive rows
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane >> 3, r = lane & 7;
    const int rr = r + kRowLanes * wave;         // first row of this lane
    const int g = blockIdx.x / tiles_n;
    const int n = (blockIdx.x % tiles_n) * 64 + 8 * c;
    const bool live = n < N;                     // N % 8 == 0: a chunk is all in or all out
    const uint16_t *wg = W + (size_t)g * G * N + (live ? n : 0);
    // The 8 columns of row k of the group (migrated when MIG).
    auto row8 = [&](int k) {
        uint4 v = load16(wg + (size_t)k * N);
        if constexpr (MIG) {
            const float ck = c_rows[(size_t)g * G + k];
            uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = ck * (float)as_half((uint16_t)u[i]);
                const float hi = ck * (float)as_half((uint16_t)(u[i] >> 16));
                u[i] = (uint32_t)as_u16((half_t)lo) | ((uint32_t)as_u16((half_t)hi) << 16);
            }
            v = make_uint4(u[0], u[1], u[2], u[3]);
        }
        return v;
    };

    // Column pairs (2 i, 2 i + 1) as half2: minimum, maximum, maximum of |w|.
    half2_t lo2[4], hi2[4], am2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo2[i] = as_half2(0x7C007C00u);   // +inf
        hi2[i] = as_half2(0xFC00FC00u);   // -inf
        am2[i] = as_half2(0u);
    }
    auto take = [&](uint4 v) {
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half2_t w2 = as_half2(u[i]);
            lo2[i] = __builtin_elementwise_min(lo2[i], w2);
            hi2[i] = __builtin_elementwise_max(hi2[i], w2);
            am2[i] = __builtin_elementwise_max(am2[i], as_half2(u[i] & 0x7FFF7FFFu));
        }
    };
    static_assert(HOLD == 0 || WPG == 1, "held rows are for one wave per group");
    uint4 hv[HOLD > 0 ? HOLD : 1][8];
    if (live) {
        if constexpr (HOLD > 0) {
#pragma unroll
            for (int h = 0; h < HOLD; ++h)
#pragma unroll
                for (int j = 0; j < 8; ++j) hv[h][j] = row8(8 * (r + 8 * h) + j);
#pragma unroll
            for (int h = 0; h < HOLD; ++h)
#pragma unroll
                for (int j = 0; j < 8; ++j) take(hv[h][j]);
        } else {
            int k = rr;
            for (; k + 7 * kStride < G; k += 8 * kStride) {
                uint4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = row8(k + u * kStride);
#pragma unroll
                for (int u = 0; u < 8; ++u) take(v[u]);
            }
            for (; k < G; k += kStride) take(row8(k));
        }
    }
    // The chunk's eight row lanes are lanes 8 c .. 8 c + 7 of each wave.
    auto hmin = [](uint32_t a, uint32_t b) { return as_u32(__builtin_elementwise_min(as_half2(a), as_half2(b))); };
    auto hmax = [](uint32_t a, uint32_t b) { return as_u32(__builtin_elementwise_max(as_half2(a), as_half2(b))); };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo2[i] = as_half2(lane_group_reduce<kRowLanes>(as_u32(lo2[i]), hmin));
        hi2[i] = as_half2(lane_group_reduce<kRowLanes>(as_u32(hi2[i]), hmax));
        am2[i] = as_half2(lane_group_reduce<kRowLanes>(as_u32(am2[i]), hmax));
    }
    if constexpr (WPG > 1) {
        __shared__ uint32_t part[WPG][8][3][4];   // wave, chunk, quantity, column pair
        if (r == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                part[wave][c][0][i] = as_u32(lo2[i]);
                part[wave][c][1][i] = as_u32(hi2[i]);
                part[wave][c][2][i] = as_u32(am2[i]);
            }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < WPG; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo2[i] = __builtin_elementwise_min(lo2[i], as_half2(part[v][c][0][i]));
                hi2[i] = __builtin_elementwise_max(hi2[i], as_half2(part[v][c][1][i]));
                am2[i] = __builtin_elementwise_max(am2[i], as_half2(part[v][c][2][i]));
            }
    }
    if (!live) return;
    float lo[8], hi[8], amax[8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            lo[2 * i + e] = (float)lo2[i][e];
            hi[2 * i + e] = (float)hi2[i][e];
            amax[2 * i + e] = (float)am2[i][e];
        }

    float sv[8], zv[8], inv[8];
    uint32_t sh[4] = {0u, 0u, 0u, 0u}, zword = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        double rg;
        if (SYM) {
            rg = (double)amax[i] / 7.0;
        } else {
            double range = (double)hi[i] - (double)lo[i];
            if (range == 0.0) range = fabs((double)hi[i]);
            rg = range / 15.0;
        }
        uint16_t s16 = f64_to_f16_rne(rg);
        if ((s16 & 0x7FFFu) == 0u) s16 = 0x3C00u;   // 1.0
        sv[i] = (float)as_half(s16);
        inv[i] = 1.0f / sv[i];
        zv[i] = SYM ? 8.0f : clamp_code(__builtin_rintf(-lo[i] / sv[i]));
        sh[i / 2] |= (uint32_t)s16 << (16 * (i % 2));
        zword |= (uint32_t)zv[i] << (4 * i);
    }
    if (rr == 0) {
        *reinterpret_cast<uint4 *>(S + (size_t)g * N + n) = make_uint4(sh[0], sh[1], sh[2], sh[3]);
        if (!SYM) QZ[(size_t)g * (N / 8) + n / 8] = zword;
    }

    // Codes of packed row p (its eight rows in v) as the chunk's eight words.
    auto emit = [&](int p, const uint4 (&v)[8]) {
        // Value of column i in row j of the packed row.
        auto wat = [&](int j, int i) {
            const uint32_t u = i < 2 ? v[j].x : i < 4 ? v[j].y : i < 6 ? v[j].z : v[j].w;
            return (float)as_half((uint16_t)(u >> (16 * (i & 1))));
        };
        uint32_t word[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                word[i] |= (uint32_t)clamp_code(rint_quotient(wat(j, i), sv[i], inv[i]) + zv[i]) << (4 * j);
        uint32_t *qrow = Q + (size_t)(g * (G / 8) + p) * N + n;
        reinterpret_cast<uint4 *>(qrow)[0] = make_uint4(word[0], word[1], word[2], word[3]);
        reinterpret_cast<uint4 *>(qrow)[1] = make_uint4(word[4], word[5], word[6], word[7]);
    };
    if constexpr (HOLD > 0) {
#pragma unroll
        for (int h = 0; h < HOLD; ++h) emit(r + 8 * h, hv[h]);
    } else {
        for (int p = rr; p < G / 8; p += kStride) {
            uint4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = row8(8 * p + j);
            emit(p, v);
        }
    }
}

}  // namespace

template <int WPG, int HOLD, bool MIG>
hipError_t launch_q(const uint16_t *w, const float *c, uint32_t *q, uint16_t *scales, uint32_t *z, int K,
                    int N, int G, int tiles_n, long long blocks, bool symmetric, hipStream_t s) {
    if (symmetric)
        hipLaunchKernelGGL((quantize_kernel<true, WPG, HOLD, MIG>), dim3((unsigned)blocks), dim3(64 * WPG),
                           0, s, w, q, scales, z, K, N, G, tiles_n, c);
    else
        hipLaunchKernelGGL((quantize_kernel<false, WPG, HOLD, MIG>), dim3((unsigned)blocks), dim3(64 * WPG),
                           0, s, w, q, scales, z, K, N, G, tiles_n, c);
    return hipGetLastError();
}

template <bool MIG>
hipError_t launch_quantize_any(const uint16_t *w, const float *c, int32_t *qweight, uint16_t *scales,
                               int32_t *qzeros, int K, int N, int G, bool symmetric, hipStream_t s) {
    const int tiles_n = (N + 63) / 64;
    const long long blocks = (long long)(K / G) * tiles_n;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    auto *q = reinterpret_cast<uint32_t *>(qweight);
    auto *z = reinterpret_cast<uint32_t *>(qzeros);
    // Groups of 64, 128 or 256 rows: read once, held in registers between the passes.
    if (G == 64) return launch_q<1, 1, MIG>(w, c, q, scales, z, K, N, G, tiles_n, blocks, symmetric, s);
    if (G == 128) return launch_q<1, 2, MIG>(w, c, q, scales, z, K, N, G, tiles_n, blocks, symmetric, s);
    if (G == 256) return launch_q<1, 4, MIG>(w, c, q, scales, z, K, N, G, tiles_n, blocks, symmetric, s);
    // One wave per (group, 64 columns) where there are tiles enough.  Long
    // groups (1024 rows or more) with too few tiles to fill the GPU several
    // times over are read by 4, 8 or 16 waves: about 32 rows per lane, and
    // twice the waves where the tiles alone give fewer than 4096 (a 70B layer
    // with one group per column, 8192 x 28672: 257 us with 4 waves, 230 us
    // with 16; 4096 x 14336 in groups of 1024: 58 us with 4, 53 us with 8).
    if (blocks >= 4096 || G < 1024)
        return launch_q<1, 0, MIG>(w, c, q, scales, z, K, N, G, tiles_n, blocks, symmetric, s);
    // (The migrating form stops at 8 waves: at 16 its registers overflow.)
    int wpg = G >= 4096 ? 16 : G >= 2048 ? 8 : 4;
    if (wpg < 16 && blocks * wpg < 4096) wpg *= 2;
    if constexpr (!MIG)
        if (wpg == 16) return launch_q<16, 0, MIG>(w, c, q, scales, z, K, N, G, tiles_n, blocks, symmetric, s);
    if (wpg >= 8) return launch_q<8, 0, MIG>(w, c, q, scales, z, K, N, G, tiles_n, blocks, symmetric, s);
    return launch_q<4, 0, MIG>(w, c, q, scales, z, K, N, G, tiles_n, blocks, symmetric, s);
}

hipError_t launch_quantize(const uint16_t *w, int32_t *qweight, uint16_t *scales, int32_t *qzeros,
                           int K, int N, int G, bool symmetric, hipStream_t s) {
    return launch_quantize_any<false>(w, nullptr, qweight, scales, qzeros, K, N, G, symmetric, s);
}

hipError_t launch_quantize_migrated(const uint16_t *w, const float *c, int32_t *qweight,
                                    uint16_t *scales, int32_t *qzeros, int K, int N, int G,
                                    bool symmetric, hipStream_t s) {
    return launch_quantize_any<true>(w, c, qweight, scales, qzeros, K, N, G, symmetric, s);
}

}  // namespace awq
