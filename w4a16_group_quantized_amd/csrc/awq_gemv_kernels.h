// Kernels of the fused W4A16 dequantize-and-multiply for small batches
// (1 <= M <= 16): the decode-time matrix-vector product of AWQ's WQLinear_GEMV module (pyshine.com
// AutoAWQ tour, overview bullets; unfragile.ai AutoAWQ page, the WQLinear
// paragraph: INT4 weights dequantized on the fly, fp16 weights never written).
//
// Bound: HBM.  Every packed weight byte is read exactly once per call, in
// coalesced 16-byte loads; scales and zero points once per group; X and Y are
// small.  Two things decide the speed:
//
// 1. Bytes in flight.  A 30 MB weight streams in ~4 us at 8 TB/s, barely more
//    than a few memory latencies, so each wave keeps D segments (SEGR packed
//    rows each) of loads in flight and issues them with no branch between them
//    (out-of-range lanes read a clamped, in-bounds address and their results
//    are dropped at the end).
//
// 2. ALU work per packed word.  At 8 TB/s the vector units have ~20 lane-ops
//    per 32-bit word, so codes are never converted to weights one by one:
//    * nibbles become fp16 biased values (1024 + q, or 64 + q for the upper
//      nibble of a byte) with one shift and four AND-ORs per word;
//    * the multiply runs on the matrix cores (v_mfma_f32_16x16x32_f16): one
//      packed word is exactly one lane's B operand (8 k of one column) and the
//      rows of X fill the A operand, so M = 1 and M = 16 cost the same ALU
//      work per weight (A rows beyond M repeat row M-1 and are never stored);
//    * the bias and zero point are removed once per group segment, not per
//      weight: with C = sum_k a (biased value) over the segment, the staged or
//      computed sums U and S give s * (C - U - z S) = s * sum_k x (q - z), two
//      FMAs per output.
//
// Kernels:
//   stream_kernel (M <= 16, G a multiple of 128): each wave stages the slice
//     of X its K range needs into its own LDS region, odd k divided by 16 so
//     that the 64-biased upper nibbles need no shift; no workgroup barrier
//     before the loop.  Up to four rows the slice is staged before the first
//     multiply (X must fit LDS), together with the per-segment sums U and S;
//     beyond four, each segment's part is loaded with that segment's weights
//     and staged into a one-segment slot just before it is multiplied, so any
//     K fits (also up to four rows when X exceeds LDS), and U and S come from
//     two more MFMAs per step against constant B operands;
//   fold_kernel (G a multiple of 32, for shapes the stream kernel does not
//     take: G not a multiple of 128, or K below 1024): the same fold, with X
//     from LDS or L2 and S from an MFMA against an all-ones B;
//   exact_kernel (any other G): every word dequantized exactly first.
//
// Tiling: one workgroup owns TN = 16 * WPL columns and all of K.  Each lane
// loads WPL consecutive words (columns) of one packed row; lanes 16j..16j+15
// take packed row 4t + j of step t, so a step covers 32 k.  The NW waves split
// K into contiguous ranges of whole 128-k segments (when the segment count is
// not a multiple of the waves, the first waves take one more); their fp32
// partial sums are added in LDS in a fixed order (deterministic) and written
// as fp16.
//
// This header holds the kernels and their launch templates; each
// awq_gemv_*.hip file instantiates one family of them (so that every kernel
// is compiled in exactly one translation unit, and the units build in
// parallel), and awq_gemv.hip picks the kernel for a shape.
#pragma once

#include "awq_device.h"
#include "awq_timeline.h"
#include "awq_internal.h"

namespace awq {
namespace gemv {

template <int WPL>
struct Words {
    uint32_t w[WPL];
};

template <int WPL>
__device__ __forceinline__ Words<WPL> load_words(const uint32_t *p) {
    Words<WPL> r;
    if constexpr (WPL == 1) {
        r.w[0] = __builtin_nontemporal_load(p);
    } else if constexpr (WPL == 2) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        r.w[0] = v.x;
        r.w[1] = v.y;
    } else {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < WPL / 4; ++i) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + i);
            r.w[4 * i + 0] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    }
    return r;
}

// Buffer descriptor over [base, base + bytes): raw (unstructured) access, the
// offsets split into a per-lane part (VGPR) and a wave-uniform part (SGPR), so
// no per-load 64-bit address arithmetic is needed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

template <int WPL>
__device__ __forceinline__ Words<WPL> buffer_words(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    Words<WPL> r;
    if constexpr (WPL == 1) {
        r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
    } else if constexpr (WPL == 2) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
        r.w[0] = v.x;
        r.w[1] = v.y;
    } else {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < WPL / 4; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * i, soff, 0);
            r.w[4 * i + 0] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    }
    return r;
}

// WPL consecutive fp16 scales, packed two per dword.
template <int WPL>
struct Scales {
    uint32_t h[(WPL + 1) / 2];
};

template <int WPL>
__device__ __forceinline__ Scales<WPL> load_scales(const uint16_t *p) {
    Scales<WPL> r;
    if constexpr (WPL == 1) {
        r.h[0] = p[0];
    } else if constexpr (WPL == 2) {
        r.h[0] = *reinterpret_cast<const uint32_t *>(p);
    } else if constexpr (WPL == 4) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        r.h[0] = v.x;
        r.h[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < WPL / 8; ++i) {
            const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
            r.h[4 * i + 0] = v.x;
            r.h[4 * i + 1] = v.y;
            r.h[4 * i + 2] = v.z;
            r.h[4 * i + 3] = v.w;
        }
    }
    return r;
}

template <int WPL>
__device__ __forceinline__ Scales<WPL> buffer_scales(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    Scales<WPL> r;
    if constexpr (WPL == 1) {
        r.h[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0);
    } else if constexpr (WPL == 2) {
        r.h[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
    } else if constexpr (WPL == 4) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
        r.h[0] = v.x;
        r.h[1] = v.y;
    } else {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < WPL / 8; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * i, soff, 0);
            r.h[4 * i + 0] = v.x;
            r.h[4 * i + 1] = v.y;
            r.h[4 * i + 2] = v.z;
            r.h[4 * i + 3] = v.w;
        }
    }
    return r;
}

template <int WPL>
__device__ __forceinline__ float scale_at(const Scales<WPL> &s, int i) {
    return (float)as_half((uint16_t)(s.h[i / 2] >> (16 * (i % 2))));
}

__device__ __forceinline__ half8_t as_b(const uint32_t p[4]) {
    return as_half8(make_uint4(p[0], p[1], p[2], p[3]));
}

// X staged in LDS row-major, K / 8 chunks per row: chunk r of row m sits at
// r ^ (m % 16) when K / 8 is a multiple of 16, so that one chunk of 16
// different rows (an A-operand read of 16 lanes) falls in 16 bank groups.
__device__ __forceinline__ int xlds_swizzle(int m, int K) { return (K & 127) == 0 ? (m & 15) : 0; }

// The A operand of one step: row xrow of X, packed row r (k = 8r .. 8r+7).
template <bool XLDS>
__device__ __forceinline__ half8_t load_a(const uint16_t *__restrict__ X, const uint4 *xs, int xrow,
                                         int K, int r) {
    if constexpr (XLDS) return as_half8(xs[xrow * (K / 8) + (r ^ xlds_swizzle(xrow, K))]);
    else return as_half8(natural_to_pairs(
             reinterpret_cast<const uint4 *>(X + (size_t)xrow * K)[r]));
}

// The loads of one segment (SEGR packed rows of WPL columns), held in registers.
template <int WPL, int STEPS>
struct Seg {
    Words<WPL> q[STEPS];
    Scales<WPL> sc;
    uint32_t zw;
};

// X up to this many bytes is staged in LDS (with the reduction buffer the
// workgroup stays within 64 KB of LDS).
constexpr size_t kXLdsBytes = 32 * 1024;

// Live rows of the 16x16 MFMA output per lane: lane (kb, c16) holds rows
// 4 kb + v, v < 4, and rows at or beyond M are never stored, so for M = 1 and
// M = 2 only v < M needs the per-segment correction.
constexpr int live_rows(int M) { return M >= 3 ? 4 : M; }

// Folded path: G is a multiple of 32; SEGR packed rows (8 * SEGR k) per segment,
// SEGR a multiple of 4 dividing G / 8.  The NW waves split the nseg segments of
// K evenly (the launcher makes nseg a multiple of NW and the per-wave count a
// multiple of D).  Each wave keeps D segments in flight: the loads of segment
// s + D are issued right after segment s has been multiplied, into the
// registers it freed.  Every load is unconditional, so the compiler can count
// outstanding loads exactly and wait for the oldest segment only.
template <int WPL, int NW, int SEGR, int D, int VR, bool SYM, bool XLDS>
__global__ void __launch_bounds__(NW * 64)
fold_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ Q,
            const uint16_t *__restrict__ S, const uint32_t *__restrict__ QZ,
            uint16_t *__restrict__ Y, int M, int K, int N, int G, int il) {
    constexpr int TN = 16 * WPL;
    constexpr int STEPS = SEGR / 4;
    constexpr int XMAX = (int)(kXLdsBytes / 16) / (NW * 64);   // X chunks per thread
    extern __shared__ __attribute__((aligned(16))) uint4 lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15;   // column block of B, row of A, column of C
    const int kb = lane >> 4;    // which packed row of a step
    const int n0 = blockIdx.x * TN;
    const int ncol = n0 + WPL * c16;
    const int ncl = ncol < N ? ncol : N - WPL;   // clamped: in bounds, result dropped
    const int xrow = c16 < M ? c16 : M - 1;      // clamped: row never stored
    const int KR = K / 8;
    const int per = KR / SEGR / NW;              // segments per wave, a multiple of D
    const int s_begin = wave * per;

    // Lane offsets (column, row within the step) in VGPRs; row and group
    // offsets, which are wave-uniform, in SGPRs.
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q, (uint32_t)KR * (uint32_t)N * 4u);
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(S, (uint32_t)(K / G) * (uint32_t)N * 2u);
    const __amdgpu_buffer_rsrc_t zrs = make_rsrc(QZ, SYM ? 0u : (uint32_t)(K / G) * (uint32_t)N / 2u);
    // il: the qweight layout (nonzero: interleaved nibble order; 2: blocked).
    const bool blk = il == 2;
    const int qp = q_pitch(blk, N);
    const int qvoff = (int)(q_col(blk, ncl, KR) + (uint32_t)(kb * qp)) * 4;
    const int svoff = ncl * 2;
    const int zvoff = (ncl / 8) * 4;
    const int zshift = 4 * (ncl % 8);
    const int xchunks = XLDS ? M * (K / 8) : 0;
    float *red = reinterpret_cast<float *>(lds + xchunks);
    const uint4 *xs = lds;

    auto load_seg = [&](int seg, Seg<WPL, STEPS> &b) {
        const int r0 = seg * SEGR;
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
            b.q[st] = buffer_words<WPL>(qrs, qvoff, (r0 + 4 * st) * qp * 4);
        const int g = (8 * r0) / G;
        b.sc = buffer_scales<WPL>(srs, svoff, g * N * 2);
        if constexpr (!SYM) b.zw = __builtin_amdgcn_raw_buffer_load_b32(zrs, zvoff, g * (N / 8) * 4, 0);
    };

    const half8_t ones = as_half8(make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
    const uint32_t nmask = nibble_mask_vgpr();
    float acc[WPL][VR];
#pragma unroll
    for (int i = 0; i < WPL; ++i)
#pragma unroll
        for (int v = 0; v < VR; ++v) acc[i][v] = 0.f;

    auto compute_seg = [&](int seg, const Seg<WPL, STEPS> &b) {
        const int r0 = seg * SEGR;
        float4_t C[WPL];
#pragma unroll
        for (int i = 0; i < WPL; ++i) C[i] = float4_t{0.f, 0.f, 0.f, 0.f};
        float4_t Cs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const half8_t a = load_a<XLDS>(X, xs, xrow, K, r0 + 4 * st + kb);
#pragma unroll
            for (int i = 0; i < WPL; ++i) {
                uint32_t p[4];
                unpack_biased(il ? deinterleave_word(b.q[st].w[i]) : b.q[st].w[i], nmask, p);
                C[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, as_b(p), C[i], 0, 0, 0);
            }
            Cs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ones, Cs, 0, 0, 0);
        }
        const uint32_t zw = SYM ? 0u : b.zw >> zshift;
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const float s = scale_at<WPL>(b.sc, i);
            const float bz = SYM ? 1032.f : 1024.f + (float)((zw >> (4 * i)) & 0xFu);
#pragma unroll
            for (int v = 0; v < VR; ++v)
                acc[i][v] = __builtin_fmaf(s, __builtin_fmaf(-bz, Cs[v], C[i][v]), acc[i][v]);
        }
    };

    // X loads first (clamped, so unconditional), then the first D segments: X
    // (an L2 hit) arrives while the weight loads are still in flight.
    Seg<WPL, STEPS> b[D];
    uint4 xr[XMAX > 0 ? XMAX : 1];
    if constexpr (XLDS) {
#pragma unroll
        for (int j = 0; j < XMAX; ++j) {
            const int c = threadIdx.x + j * NW * 64;
            xr[j] = reinterpret_cast<const uint4 *>(X)[c < xchunks ? c : 0];
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) load_seg(s_begin + d, b[d]);
    if constexpr (XLDS) {
#pragma unroll
        for (int j = 0; j < XMAX; ++j) {
            const int c = threadIdx.x + j * NW * 64;
            const int m = c / (K / 8), r = c - m * (K / 8);
            if (c < xchunks) lds[m * (K / 8) + (r ^ xlds_swizzle(m, K))] = natural_to_pairs(xr[j]);
        }
        __syncthreads();
    }

    for (int i = 0; i < per - D; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            compute_seg(s_begin + i + d, b[d]);
            load_seg(s_begin + i + d + D, b[d]);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) compute_seg(s_begin + per - D + d, b[d]);

    // C layout of the 16x16 MFMA: lane (kb, c16) holds rows 4 kb + v of column c16.
    __syncthreads();   // every wave is done with the staged X and the tables
#pragma unroll
    for (int v = 0; v < VR; ++v) {
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

// ---------------------------------------------------------------------------
// Small batches (M <= 16, X staged in LDS), the decode case.
//
// Each wave stages the rows of X that its K range needs in its own LDS slice
// (no workgroup barrier), each 8-k chunk already in the k order of the
// unpacked weights, with the odd k divided by 16 (exact in fp16 above 2^-10):
//     A chunk = (x0, x4, x1/16, x5/16, x2, x6, x3/16, x7/16).
// That lets one shift and four AND-ORs unpack a word:
//     (w & 0x000F000F)      | bias = (1024 + q0,    1024 + q4)
//     (w & 0x00F000F0)      | bias = (1024 + 16 q1, 1024 + 16 q5)
//     (w>>8 & 0x000F000F)   | bias = (1024 + q2,    1024 + q6)
//     (w>>8 & 0x00F000F0)   | bias = (1024 + 16 q3, 1024 + 16 q7)
// and the products against A come out as x_j (1024 + q_j) for even k and
// (x_j / 16)(1024 + 16 q_j) = 64 x_j + x_j q_j for odd k.  With
//     U = 1024 * sum_k a_k   (a_k the staged A values)
//     S = sum_even x + 16 * sum_odd (x/16)   (= sum_k x)
// a group's MFMA sum C gives sum_k x (q - z) = C - U - z S.  U and S per row
// and segment are computed once, while staging, so no MFMA is spent on them.
// ---------------------------------------------------------------------------

constexpr uint32_t kSixteenthX2 = 0x2C002C00u;   // (1/16, 1/16) in fp16


__device__ __forceinline__ void unpack_biased16(uint32_t w, uint32_t lo_mask, uint32_t hi_mask,
                                                uint32_t p[4]) {
    const uint32_t w8 = w >> 8;
    p[0] = (w & lo_mask) | kBias1024x2;
    p[1] = (w & hi_mask) | kBias1024x2;
    p[2] = (w8 & lo_mask) | kBias1024x2;
    p[3] = (w8 & hi_mask) | kBias1024x2;
}

// Natural-order chunk of X -> staged A chunk (see above).
__device__ __forceinline__ uint4 stage_chunk(uint4 x) {
    uint4 a = natural_to_pairs(x);
    a.y = as_u32(as_half2(a.y) * as_half2(kSixteenthX2));
    a.w = as_u32(as_half2(a.w) * as_half2(kSixteenthX2));
    return a;
}

template <int WPL, int STEPS, bool SYM>
struct WSeg {
    Words<WPL> q[STEPS];
    Scales<WPL> sc;
    uint32_t zw, zw2;   // zw2: zero word of the up columns (fused gate/up only)
};

// Two half-width loads side by side (fused gate/up: gate columns, up columns).
template <int WPL>
__device__ __forceinline__ Words<WPL> join(const Words<WPL / 2> &a, const Words<WPL / 2> &b) {
    Words<WPL> r;
#pragma unroll
    for (int i = 0; i < WPL / 2; ++i) {
        r.w[i] = a.w[i];
        r.w[WPL / 2 + i] = b.w[i];
    }
    return r;
}
template <int WPL>
__device__ __forceinline__ Scales<WPL> join(const Scales<WPL / 2> &a, const Scales<WPL / 2> &b) {
    Scales<WPL> r;
#pragma unroll
    for (int i = 0; i < WPL / 4; ++i) {
        r.h[i] = a.h[i];
        r.h[WPL / 4 + i] = b.h[i];
    }
    return r;
}

// SiLU in fp32: t / (1 + e^-t); far below zero the quotient is a signed zero.
__device__ __forceinline__ float silu(float t) { return t / (1.0f + __expf(-t)); }

// Whether the segment-by-segment kernel gives its reduction buffer LDS of its
// own (beside the X slots, instead of over them): 128 columns per workgroup
// and more than 8 rows.
__host__ __device__ __forceinline__ bool sep_reduction(int M, int WPL) { return WPL == 8 && M > 8; }

// Chunks of staged X per lane, at most.
constexpr int kStageChunks = 16;
// LDS of one workgroup, at most (gfx950: 160 KB per workgroup).
constexpr size_t kLdsMax = 160 * 1024;

// XCH: 16-byte chunks of X each lane stages (the largest wave's slice,
// M * ceil(segments / NW) * SEGR chunks, is at most 64 * XCH).
// GU 1 (fused gate/up): the layer's N columns are [gate | up]; a lane's WPL words
// are WPL / 2 gate columns and the same WPL / 2 columns of the up half, and the
// output is h = fp16(SiLU(gate) * up), N / 2 columns wide.  GU 2 (paired
// strips, a plain layer with N a multiple of 16): the same loads, a workgroup
// taking a strip of each half of the columns, and the plain output y.
// XS > 0 stages X progressively: the XS chunks per lane of a segment's slice
// of X (M * SEGR <= 64 * XS) are loaded with the segment's weights and staged
// just before the segment is multiplied, instead of the whole slice up front.
// With 16 rows the whole slice is 128 KB per workgroup, and every workgroup
// asking for it at once delays the first multiply by microseconds.
// IL: the qweight layout (0 canonical, 1 interleaved, 2 blocked; awq_repack).
// Nonzero: interleaved nibble order.  A word then unpacks into the natural-order pairs (k 2e,
// k 2e + 1) as (1024 + q, 1024 + q') for even e and (64 + q, 64 + q') for odd
// e, so X is staged in natural order with no x / 16, and the bias sum U weighs
// the odd pairs' x by 64 instead of 1024.  2: the words of a workgroup's strip
// are one contiguous run per 128-column block (q_col, q_pitch).
// UNEV: the K range's segments do not split into whole pipelines of D per
// wave (K not a multiple of 8 NW SEGR, or an odd count per wave): the first
// nseg % NW waves take one segment more, and the loads ahead are guarded by
// the wave's own count (a uniform branch).  The even case keeps the
// unconditional pipeline.
template <int WPL, int NW, int SEGR, int D, int VR, bool SYM, bool GRP1, int XCH, int GU = 0,
          int XS = 0, bool UNEV = false, int IL = 0>
__global__ void __launch_bounds__(NW * 64)
stream_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ Q,
              const uint16_t *__restrict__ S, const uint32_t *__restrict__ QZ,
              uint16_t *__restrict__ Y, int M, int K, int N, int G) {
    AWQ_TL_STAMP(tl_start);
    AWQ_TL_CLOCK(tc_start);
    constexpr int TN = 16 * WPL;              // weight columns (MFMA column slots) per workgroup
    constexpr int WO = GU ? WPL / 2 : WPL;    // output columns per lane
    constexpr int TO = 16 * WO;               // output columns per workgroup
    constexpr int STEPS = SEGR / 4;
    extern __shared__ __attribute__((aligned(16))) uint4 lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15;   // column block of B, row of A, column of C
    const int kb = lane >> 4;    // packed row within a step; C rows 4 kb .. 4 kb + 3
    const int NO = GU ? N / 2 : N;               // output width
    const int n0 = blockIdx.x * TO;
    const int ncol = n0 + WO * c16;
    const int ncl = ncol < NO ? ncol : NO - WO;  // clamped: in bounds, result dropped
    const int KR = K / 8;
    const int nseg = KR / SEGR;
    const int per_base = nseg / NW, extra = UNEV ? nseg % NW : 0;
    const int per = per_base + (wave < extra ? 1 : 0);   // this wave's segments
    const int tper = per_base + (extra > 0 ? 1 : 0);     // stride of the per-wave regions
    const int rows_w = per * SEGR;               // packed rows of this wave
    const int s_begin = wave * per_base + (wave < extra ? wave : extra);
    const int r_begin = s_begin * SEGR;
    const int spg = G / (8 * SEGR);              // segments per group

    // LDS: staged X slices (all waves), then (U, S) tables; once every wave is
    // done with them, the reduction buffer takes their place.  Chunk rr of row
    // m of a slice sits at rr ^ (m % 16) (rows_w is a multiple of 16, so the
    // chunk stays in its row): an A-operand read takes one chunk of 16
    // different rows per 16 lanes, which then fall in 16 different bank groups
    // instead of one.
    // Progressive staging keeps one segment's slot per wave: a wave stages a
    // segment right before multiplying it, after its reads of the previous one
    // (a wave's LDS operations execute in order), so one slot suffices and the
    // kernel takes any K.  Otherwise the wave's whole slice is staged.
    constexpr bool SLOT = XS > 0;
    const int XR = SLOT ? SEGR : tper * SEGR;    // staged chunks per row of a wave's region
    uint4 *xs = lds + wave * (M * XR);
    float2 *tabs = reinterpret_cast<float2 *>(lds + NW * M * XR);
    float2 *tab = tabs + wave * (M * tper);
    // Slot mode with a large reduction buffer (128 columns per workgroup, more
    // than 8 rows; stream_lds_prog sizes LDS the same way): the buffer lies after
    // the slots, so that a wave writes its partial sums as soon as its own loop
    // ends, with no barrier before.  16 rows of 4096 x 28672, two runs: 13.67-13.98
    // -> 13.50-13.53 us (awq_gemv), 13.83-13.89 -> 13.51-13.58 us (fused
    // gate/up); of 8192 x 28672: 23.47 -> 23.22 us.  At 4 to 16 rows on 64-column
    // strips, and at 4 rows on 128 columns, it cost 0.3-1.8%.
    const bool own_red = SLOT && sep_reduction(M, WPL);
    float *red = reinterpret_cast<float *>(own_red ? lds + NW * M * XR : lds);

    const int xrow = c16 < M ? c16 : M - 1;      // A row of this lane (clamped)
    constexpr bool BLK = blocked_layout(IL);
    const int qp = q_pitch(BLK, N);
    const uint32_t lane_q = q_col(BLK, ncl, KR) + (uint32_t)(kb * qp);
    const uint32_t lane_q2 = GU ? q_col(BLK, ncl + NO, KR) + (uint32_t)(kb * qp) : 0u;   // up half

    // Scale and zero of one segment; loads of one segment.
    auto load_seg = [&](int seg, WSeg<WPL, STEPS, SYM> &b) {
        const int r0 = seg * SEGR;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const uint32_t *qrow = Q + (size_t)(r0 + 4 * st) * qp;   // wave-uniform
            if constexpr (GU)
                b.q[st] = join<WPL>(load_words<WO>(qrow + lane_q), load_words<WO>(qrow + lane_q2));
            else
                b.q[st] = load_words<WPL>(qrow + lane_q);
        }
        const int g = (8 * r0) / G;
        const uint16_t *srow = S + (size_t)g * N;
        if constexpr (GU) b.sc = join<WPL>(load_scales<WO>(srow + ncl), load_scales<WO>(srow + NO + ncl));
        else b.sc = load_scales<WPL>(srow + ncl);
        if constexpr (!SYM) {
            b.zw = QZ[(size_t)g * (N / 8) + ncl / 8];
            if constexpr (GU) b.zw2 = QZ[(size_t)g * (N / 8) + (NO + ncl) / 8];
        }
    };

    // Staging of one chunk: row m, wave-local packed row rr, `live` false for
    // the padding lanes.  The segment sums (U, S) of a row are reduced over the
    // aligned groups of SEGR lanes that hold that row's chunks of one segment.
    auto stage = [&](const uint4 &raw, bool live, int m, int rr) {
        const uint4 a = IL ? raw : stage_chunk(raw);
        if constexpr (SLOT) {   // the segment sums come from the matrix cores
            if (live) xs[m * XR + ((rr % SEGR) ^ (m & 15))] = a;
            return;
        }
        const half2_t one2 = {(half_t)1.0f, (half_t)1.0f};
        const float lo = __builtin_amdgcn_fdot2(as_half2(a.x), one2,
                         __builtin_amdgcn_fdot2(as_half2(a.z), one2, 0.f, false), false);
        const float hi = __builtin_amdgcn_fdot2(as_half2(a.y), one2,
                         __builtin_amdgcn_fdot2(as_half2(a.w), one2, 0.f, false), false);
        // t: U / 1024 (the staged values weighed by their pairs' bias / 1024);
        // u: the sum of x.
        float t = live ? (IL ? lo + 0.0625f * hi : lo + hi) : 0.f;
        float u = live ? (IL ? lo + hi : lo + 16.f * hi) : 0.f;
        t = lane_group_sum<SEGR>(t);
        u = lane_group_sum<SEGR>(u);
        if (live) {
            xs[m * XR + ((SLOT ? rr % SEGR : rr) ^ (m & 15))] = a;
            if (rr % SEGR == 0) tab[m * tper + rr / SEGR] = make_float2(1024.f * t, u);
        }
    };
    // Only this wave reads its slice; LDS operations of one wave execute in order.
    auto staged = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    const uint4 *X4 = reinterpret_cast<const uint4 *>(X);
    WSeg<WPL, STEPS, SYM> b[D];
    // Progressive staging: chunk c = lane + 64 j of segment sl is row c / SEGR,
    // packed row sl * SEGR + c % SEGR of the wave's slice (clamped loads).
    // A segment's swizzled chunks (rr ^ (m % 16)) stay in its own 16 packed rows.
    static_assert(XS == 0 || SEGR % 16 == 0, "progressive staging needs 16-row segments");
    constexpr int XSN = XS > 0 ? XS : 1;
    uint4 xq[D][XSN];
    auto load_x_seg = [&](int sl, uint4 (&q)[XSN]) {
#pragma unroll
        for (int j = 0; j < XSN; ++j) {
            const int c = lane + 64 * j;
            const int cc = c < M * SEGR ? c : 0;
            q[j] = X4[(size_t)(cc / SEGR) * KR + r_begin + sl * SEGR + cc % SEGR];
        }
    };
    auto stage_x_seg = [&](int sl, const uint4 (&q)[XSN]) {
#pragma unroll
        for (int j = 0; j < XSN; ++j) {
            const int c = lane + 64 * j;
            stage(q[j], c < M * SEGR, c / SEGR, sl * SEGR + c % SEGR);
        }
        staged();
    };

    if constexpr (XS > 0) {
        // X chunks of a segment first, then its weights: the wait for the
        // chunks does not wait for the segment's own weights.
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_x_seg(d, xq[d]);
            load_seg(s_begin + d, b[d]);
        }
    } else {
        // 1. X loads (clamped, unconditional), 2. the first D segments, 3. staging.
        const int chunks_w = M * rows_w;
        uint4 xr[XCH];
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
            const int c = lane + 64 * j;
            const int cc = c < chunks_w ? c : 0;
            const int m = VR == 1 ? 0 : cc / rows_w;             // VR == 1 means M == 1
            const int rr = VR == 1 ? cc : cc - m * rows_w;
            xr[j] = X4[(size_t)m * KR + r_begin + rr];
        }
#pragma unroll
        for (int d = 0; d < D; ++d) load_seg(s_begin + d, b[d]);
#pragma unroll
        for (int j = 0; j < XCH; ++j) {
            const int c = lane + 64 * j;
            const int m = VR == 1 ? 0 : c / rows_w;
            stage(xr[j], c < chunks_w, m, c - m * rows_w);
        }
        staged();
    }

    const uint32_t lo_mask = nibble_mask_vgpr();
    const uint32_t hi_mask = high_mask_vgpr();
    float acc[WPL][VR];
#pragma unroll
    for (int i = 0; i < WPL; ++i)
#pragma unroll
        for (int v = 0; v < VR; ++v) acc[i][v] = 0.f;
    float4_t C[WPL];
#pragma unroll
    for (int i = 0; i < WPL; ++i) C[i] = float4_t{0.f, 0.f, 0.f, 0.f};
    float Ug[VR], Sg[VR];
#pragma unroll
    for (int v = 0; v < VR; ++v) Ug[v] = Sg[v] = 0.f;
    // Slot mode: the sums of the staged values (T) and of x (S) of each row,
    // over the group so far, from two more MFMAs per step against constant B
    // operands: all ones, and 1 for the even-k halves, 16 for the odd-k ones
    // (staged as x / 16).  Lane (kb, c16) receives them for its C rows 4 kb + v.
    float4_t CT = float4_t{0.f, 0.f, 0.f, 0.f}, CS = CT;
    const half8_t ones8 = as_half8(make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
    const half8_t xsum8 = as_half8(make_uint4(0x3C003C00u, 0x4C004C00u, 0x3C003C00u, 0x4C004C00u));
    // Interleaved words: U / 1024 weighs the odd pairs by 1/16; S is the plain sum.
    const half8_t tsum8 = as_half8(make_uint4(0x3C003C00u, 0x2C002C00u, 0x3C003C00u, 0x2C002C00u));

    auto compute_seg = [&](int seg, const WSeg<WPL, STEPS, SYM> &bb) {
        const int rl0 = (seg - s_begin) * SEGR;   // local packed row of the segment
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const half8_t a = as_half8(xs[xrow * XR + (((SLOT ? 0 : rl0) + 4 * st + kb) ^ (xrow & 15))]);
            if constexpr (SLOT) {
                CT = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, IL ? tsum8 : ones8, CT, 0, 0, 0);
                CS = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, IL ? ones8 : xsum8, CS, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < WPL; ++i) {
                uint32_t p[4];
                if constexpr (IL) unpack_interleaved(bb.q[st].w[i], lo_mask, hi_mask, p);
                else unpack_biased16(bb.q[st].w[i], lo_mask, hi_mask, p);
                C[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, as_b(p), C[i], 0, 0, 0);
            }
        }
        // (U, S) of this segment for the lane's live C rows 4 kb + v (clamped).
        if constexpr (!SLOT) {
#pragma unroll
            for (int v = 0; v < VR; ++v) {
                const int m = min(4 * kb + v, M - 1);
                const float2 us = tab[m * tper + (seg - s_begin)];
                Ug[v] += us.x;
                Sg[v] += us.y;
            }
        }
        const bool fold = GRP1 || (seg + 1) % spg == 0 || seg == s_begin + per - 1;   // uniform
        if (fold) {
            if constexpr (SLOT) {
#pragma unroll
                for (int v = 0; v < VR; ++v) {
                    Ug[v] = 1024.f * CT[v];
                    Sg[v] = CS[v];
                }
                CT = float4_t{0.f, 0.f, 0.f, 0.f};
                CS = CT;
            }
            const uint32_t zw = SYM ? 0u : bb.zw >> (4 * (ncl % 8));
            const uint32_t zw2 = SYM || !GU ? 0u : bb.zw2 >> (4 * (ncl % 8));   // NO % 8 == 0
#pragma unroll
            for (int i = 0; i < WPL; ++i) {
                const float sv = scale_at<WPL>(bb.sc, i);
                const uint32_t zi = GU && i >= WO ? zw2 >> (4 * (i - WO)) : zw >> (4 * i);
                const float z = SYM ? 8.f : (float)(zi & 0xFu);
#pragma unroll
                for (int v = 0; v < VR; ++v)
                    acc[i][v] = __builtin_fmaf(sv, __builtin_fmaf(-z, Sg[v], C[i][v] - Ug[v]),
                                               acc[i][v]);
                C[i] = float4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int v = 0; v < VR; ++v) Ug[v] = Sg[v] = 0.f;
        }
    };

    if constexpr (!UNEV) {
        for (int i = 0; i < per - D; i += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if constexpr (XS > 0) stage_x_seg(i + d, xq[d]);
                compute_seg(s_begin + i + d, b[d]);
                if constexpr (XS > 0) load_x_seg(i + d + D, xq[d]);
                load_seg(s_begin + i + d + D, b[d]);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if constexpr (XS > 0) stage_x_seg(per - D + d, xq[d]);
            compute_seg(s_begin + per - D + d, b[d]);
        }
    } else {
        // Segment i sits in buffer i % D; per >= D (the launcher's condition).
        int i = 0;
        for (; i + D < per; i += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if constexpr (XS > 0) stage_x_seg(i + d, xq[d]);
                compute_seg(s_begin + i + d, b[d]);
                if (i + d + D < per) {   // uniform
                    if constexpr (XS > 0) load_x_seg(i + d + D, xq[d]);
                    load_seg(s_begin + i + d + D, b[d]);
                }
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (i + d < per) {           // uniform
                if constexpr (XS > 0) stage_x_seg(i + d, xq[d]);
                compute_seg(s_begin + i + d, b[d]);
            }
        }
    }

    AWQ_TL_STAMP(tl_loop);
    AWQ_TL_CLOCK(tc_loop);
    // C layout of the 16x16 MFMA: lane (kb, c16) holds rows 4 kb + v of column c16.
    // Every wave is done with the staged X and the tables (not needed where the
    // reduction buffer has LDS of its own).
    if (!own_red) __syncthreads();
    AWQ_TL_STAMP(tl_red);
#pragma unroll
    for (int v = 0; v < VR; ++v) {
        const int m = 4 * kb + v;
        if (m < M)
#pragma unroll
            for (int i = 0; i < WPL; ++i) red[(wave * M + m) * TN + WPL * c16 + i] = acc[i][v];
    }
    __syncthreads();
    if constexpr (GU == 1) {
        for (int idx = threadIdx.x; idx < M * TO; idx += NW * 64) {
            const int m = idx / TO;
            const int c = idx % TO;
            const int slot = WPL * (c / WO) + c % WO;   // gate slot; up is WO further
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                gs += red[(w * M + m) * TN + slot];
                us += red[(w * M + m) * TN + slot + WO];
            }
            if (n0 + c < NO) Y[(size_t)m * NO + n0 + c] = as_u16((half_t)(silu(gs) * us));
        }
    } else if constexpr (GU == 2) {
        // Paired strips: slot c of the first half is column n0 + c, of the
        // second half column NO + n0 + c; each is summed over the waves in the
        // same order as an unpaired strip's.
        for (int idx = threadIdx.x; idx < M * TO; idx += NW * 64) {
            const int m = idx / TO;
            const int c = idx % TO;
            const int slot = WPL * (c / WO) + c % WO;
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                s1 += red[(w * M + m) * TN + slot];
                s2 += red[(w * M + m) * TN + slot + WO];
            }
            if (n0 + c < NO) {
                Y[(size_t)m * N + n0 + c] = as_u16((half_t)s1);
                Y[(size_t)m * N + NO + n0 + c] = as_u16((half_t)s2);
            }
        }
    } else {
        for (int idx = threadIdx.x; idx < M * TN; idx += NW * 64) {
            const int m = idx / TN;
            const int c = idx % TN;
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sum += red[(w * M + m) * TN + c];
            if (n0 + c < N) Y[(size_t)m * N + n0 + c] = as_u16((half_t)sum);
        }
    }
#ifdef AWQ_TIMELINE
    __builtin_amdgcn_s_waitcnt(0);   // the stores have completed
    AWQ_TL_STAMP(tl_end);
    if (lane == 0)
        awq_tl_record((int)blockIdx.x * NW + wave, tl_start, tl_loop, tl_red, tl_end, tc_start, tc_loop);
#endif
}

// Whether K's segments split over the NW waves in whole pipelines of D each.
inline bool stream_even(int K, int NW, int SEGR, int D) {
    const int nseg = K / 8 / SEGR;
    return nseg % NW == 0 && (nseg / NW) % D == 0;
}

// Dynamic LDS of stream_kernel: staged X and tables, or the reduction buffer
// that replaces them at the end, whichever is larger.
inline size_t stream_lds(int M, int K, int WPL, int NW, int SEGR) {
    const int per = (K / 8 / SEGR + NW - 1) / NW;   // the largest count per wave
    const size_t staged = (size_t)NW * M * per * SEGR * 16 + (size_t)NW * M * per * 8;
    const size_t red = (size_t)NW * M * 16 * WPL * 4;
    return staged > red ? staged : red;
}

// The same with X staged segment by segment (one segment's slot per wave).
inline size_t stream_lds_prog(int M, int K, int WPL, int NW, int SEGR) {
    (void)K;   // one segment's slot per wave, whatever K; no tables
    const size_t staged = (size_t)NW * M * SEGR * 16;
    const size_t red = (size_t)NW * M * 16 * WPL * 4;
    if (sep_reduction(M, WPL)) return staged + red;   // side by side
    return staged > red ? staged : red;
}

template <int WPL, int NW, int SEGR, int D, int VR, bool SYM, bool GRP1, int XCH, int GU = 0,
          int XS = 0, int IL = 0>
hipError_t launch_stream(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                         const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                         hipStream_t s) {
    constexpr int TO = GU ? 8 * WPL : 16 * WPL;   // output columns per workgroup
    const int NO = GU ? N / 2 : N;
    // The guarded pipeline of the fused gate/up kernel at depth 2 with two or
    // more X chunks per lane runs out of registers; such shapes take depth 1
    // (the dispatch checks stream_even first) and that variant is not built.
    constexpr bool kUneven = !(GU && D > 1 && XS > 1);
    auto even = stream_kernel<WPL, NW, SEGR, D, VR, SYM, GRP1, XCH, GU, XS, false, IL>;
    auto uneven = stream_kernel<WPL, NW, SEGR, D, VR, SYM, GRP1, XCH, GU, XS, kUneven, IL>;
    const bool split_uneven = !stream_even(K, NW, SEGR, D);
    if (!kUneven && split_uneven) return hipErrorNotSupported;
    auto kernel = split_uneven ? uneven : even;
    const size_t lds = XS > 0 ? stream_lds_prog(M, K, WPL, NW, SEGR) : stream_lds(M, K, WPL, NW, SEGR);
    if (lds > 64 * 1024) {
        // Beyond 64 KB a kernel must be allowed the larger allocation (once each).
        static const hipError_t raised_even = hipFuncSetAttribute(
            reinterpret_cast<const void *>(even), hipFuncAttributeMaxDynamicSharedMemorySize,
            (int)kLdsMax);
        static const hipError_t raised_uneven = hipFuncSetAttribute(
            reinterpret_cast<const void *>(uneven), hipFuncAttributeMaxDynamicSharedMemorySize,
            (int)kLdsMax);
        if (raised_even != hipSuccess) return raised_even;
        if (raised_uneven != hipSuccess) return raised_uneven;
    }
    hipLaunchKernelGGL(kernel, dim3((NO + TO - 1) / TO), dim3(NW * 64), lds, s, x,
                       reinterpret_cast<const uint32_t *>(qw), sc,
                       reinterpret_cast<const uint32_t *>(qz), y, M, K, N, G);
    return hipGetLastError();
}

// Whether stream_kernel<.., NW, SEGR, D, ..> can take this shape: every wave
// gets at least D segments (one pipeline), the largest wave's X slice fits
// kStageChunks chunks per lane, and LDS stays within the workgroup maximum.
inline bool stream_fits(int M, int K, int N, int G, int WPL, int NW, int SEGR, int D) {
    if (M > 16 || G % (8 * SEGR) != 0) return false;
    const int nseg = K / 8 / SEGR;
    if (nseg / NW < D) return false;             // every wave fills its pipeline
    const int per = (nseg + NW - 1) / NW;        // the largest count per wave
    if (M * per * SEGR > 64 * kStageChunks) return false;
    return stream_lds(M, K, WPL, NW, SEGR) <= kLdsMax;
}

// Whether the progressive kernel (16-row segments, X staged segment by
// segment) can take this shape: any K with at least D segments per wave, and
// the slots and the reduction within LDS.
inline bool stream_fits_prog(int M, int K, int N, int G, int WPL, int NW, int D) {
    if (M > 16 || G % 128 != 0) return false;
    const int nseg = K / 128;
    if (nseg / NW < D) return false;             // every wave fills its pipeline
    return stream_lds_prog(M, K, WPL, NW, 16) <= kLdsMax;
}

template <int WPL, int NW, int SEGR, int D, int VR, int XCH, int IL, int GU = 0>
hipError_t launch_stream_sg(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                            const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                            hipStream_t s) {
    const bool grp1 = G == 8 * SEGR;
    if (qz == nullptr)
        return grp1 ? launch_stream<WPL, NW, SEGR, D, VR, true, true, XCH, GU, 0, IL>(x, qw, sc, qz, y, M, K, N, G, s)
                    : launch_stream<WPL, NW, SEGR, D, VR, true, false, XCH, GU, 0, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    return grp1 ? launch_stream<WPL, NW, SEGR, D, VR, false, true, XCH, GU, 0, IL>(x, qw, sc, qz, y, M, K, N, G, s)
                : launch_stream<WPL, NW, SEGR, D, VR, false, false, XCH, GU, 0, IL>(x, qw, sc, qz, y, M, K, N, G, s);
}

template <int WPL, int NW, int SEGR, int D, int VR, int IL, int GU = 0>
hipError_t launch_stream_x(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                           const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                           hipStream_t s) {
    const int chunks_w = M * ((K / 8 / SEGR + NW - 1) / NW) * SEGR;   // the largest wave's
    if (chunks_w <= 64) return launch_stream_sg<WPL, NW, SEGR, D, VR, 1, IL, GU>(x, qw, sc, qz, y, M, K, N, G, s);
    if (chunks_w <= 128) return launch_stream_sg<WPL, NW, SEGR, D, VR, 2, IL, GU>(x, qw, sc, qz, y, M, K, N, G, s);
    if (chunks_w <= 256) return launch_stream_sg<WPL, NW, SEGR, D, VR, 4, IL, GU>(x, qw, sc, qz, y, M, K, N, G, s);
    if (chunks_w <= 512) return launch_stream_sg<WPL, NW, SEGR, D, VR, 8, IL, GU>(x, qw, sc, qz, y, M, K, N, G, s);
    return launch_stream_sg<WPL, NW, SEGR, D, VR, kStageChunks, IL, GU>(x, qw, sc, qz, y, M, K, N, G, s);
}

// Compute units of the current device (queried once per process).
inline int device_cus() {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return 256;
        return n;
    }();
    return cus;
}

// Beyond four rows (all four C rows of a lane live), X staged progressively:
// XS = ceil(M * 16 / 64) chunks per lane per 16-row segment.
template <int WPL, int NW, int D, int GU, int XS, int IL>
hipError_t launch_stream_prog_xs(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                                 const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                                 hipStream_t s) {
    const bool grp1 = G == 8 * 16;
#define AWQ_PROG(SYMV, GRPV) \
    launch_stream<WPL, NW, 16, D, 4, SYMV, GRPV, 1, GU, XS, IL>(x, qw, sc, qz, y, M, K, N, G, s)
    if (qz == nullptr) return grp1 ? AWQ_PROG(true, true) : AWQ_PROG(true, false);
    return grp1 ? AWQ_PROG(false, true) : AWQ_PROG(false, false);
#undef AWQ_PROG
}

template <int WPL, int NW, int D, int GU, int IL>
hipError_t launch_stream_prog(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                              const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                              hipStream_t s) {
    if (M <= 4) return launch_stream_prog_xs<WPL, NW, D, GU, 1, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    if (M <= 8) return launch_stream_prog_xs<WPL, NW, D, GU, 2, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    if (M <= 12) return launch_stream_prog_xs<WPL, NW, D, GU, 3, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    return launch_stream_prog_xs<WPL, NW, D, GU, 4, IL>(x, qw, sc, qz, y, M, K, N, G, s);
}

template <int WPL, int NW, int SEGR, int D, int IL, int GU = 0>
hipError_t launch_stream_m(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                           const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                           hipStream_t s) {
    switch (live_rows(M)) {
    case 1: return launch_stream_x<WPL, NW, SEGR, D, 1, IL, GU>(x, qw, sc, qz, y, M, K, N, G, s);
    case 2: return launch_stream_x<WPL, NW, SEGR, D, 2, IL, GU>(x, qw, sc, qz, y, M, K, N, G, s);
    default: return launch_stream_x<WPL, NW, SEGR, D, 4, IL, GU>(x, qw, sc, qz, y, M, K, N, G, s);
    }
}

// Exact path, any G (multiple of 8): every word is dequantized bit-exactly to
// fp16 (w = fp16_rne(s (q - z))) and multiplied; no per-segment correction.
template <int WPL, int NW>
__global__ void __launch_bounds__(NW * 64)
exact_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ Q,
             const uint16_t *__restrict__ S, const uint32_t *__restrict__ QZ,
             uint16_t *__restrict__ Y, int M, int K, int N, int G, int il) {
    constexpr int TN = 16 * WPL;
    extern __shared__ __attribute__((aligned(16))) uint4 lds[];
    float *red = reinterpret_cast<float *>(lds);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c16 = lane & 15;
    const int kb = lane >> 4;
    const int n0 = blockIdx.x * TN;
    const int ncol = n0 + WPL * c16;
    const int ncl = ncol < N ? ncol : N - WPL;
    const int xrow = c16 < M ? c16 : M - 1;
    const int KR = K / 8;
    const uint32_t nmask = nibble_mask_vgpr();
    const bool blk = il == 2;   // il: the qweight layout (nonzero: interleaved nibbles)
    const int qp = q_pitch(blk, N);
    const uint32_t qc = q_col(blk, ncl, KR);

    float4_t C[WPL];
#pragma unroll
    for (int i = 0; i < WPL; ++i) C[i] = float4_t{0.f, 0.f, 0.f, 0.f};
    const int nstep = (KR + 3) / 4;
    for (int st = wave; st < nstep; st += NW) {
        const int r = 4 * st + kb;
        uint32_t d[WPL][4];
        uint4 xa = make_uint4(0u, 0u, 0u, 0u);
        if (r < KR) {
            xa = reinterpret_cast<const uint4 *>(X + (size_t)xrow * K)[r];
            const Words<WPL> q = load_words<WPL>(Q + (size_t)r * qp + qc);
            const int g = (8 * r) / G;
            const uint32_t zw = QZ ? QZ[(size_t)g * (N / 8) + ncl / 8] >> (4 * (ncl % 8))
                                   : 0x88888888u;
            const uint16_t *sp = S + (size_t)g * N + ncl;
#pragma unroll
            for (int i = 0; i < WPL; ++i) {
                const half_t bz = biased_zero(zw >> (4 * i));
                const half_t sv = as_half(sp[i]);
                const half2_t bz2 = {bz, bz}, s2 = {sv, sv};
                uint32_t p[4];
                unpack_biased(il ? deinterleave_word(q.w[i]) : q.w[i], nmask, p);
#pragma unroll
                for (int j = 0; j < 4; ++j) d[i][j] = dequant_pair(p[j], bz2, s2);
            }
        } else {
#pragma unroll
            for (int i = 0; i < WPL; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) d[i][j] = 0u;
        }
        const half8_t a = as_half8(natural_to_pairs(xa));
#pragma unroll
        for (int i = 0; i < WPL; ++i)
            C[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, as_b(d[i]), C[i], 0, 0, 0);
    }

#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * kb + v;
        if (m < M)
#pragma unroll
            for (int i = 0; i < WPL; ++i) red[(wave * M + m) * TN + WPL * c16 + i] = C[i][v];
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

template <int WPL, int NW, int SEGR, int D, int VR, bool SYM, bool XLDS>
hipError_t launch_fold(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                       uint16_t *y, int M, int K, int N, int G, int il, hipStream_t s) {
    constexpr int TN = 16 * WPL;
    const size_t lds = (XLDS ? (size_t)M * K * 2 : 0) + (size_t)NW * M * TN * sizeof(float);
    hipLaunchKernelGGL((fold_kernel<WPL, NW, SEGR, D, VR, SYM, XLDS>), dim3((N + TN - 1) / TN),
                       dim3(NW * 64), lds, s, x, reinterpret_cast<const uint32_t *>(qw), sc,
                       reinterpret_cast<const uint32_t *>(qz), y, M, K, N, G, il);
    return hipGetLastError();
}

template <int WPL, int NW, int SEGR, int D, int VR>
hipError_t launch_fold_vr(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                          const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                          hipStream_t s) {
    const bool xlds = (size_t)M * K * 2 <= kXLdsBytes;
    if (qz == nullptr)
        return xlds ? launch_fold<WPL, NW, SEGR, D, VR, true, true>(x, qw, sc, qz, y, M, K, N, G, il, s)
                    : launch_fold<WPL, NW, SEGR, D, VR, true, false>(x, qw, sc, qz, y, M, K, N, G, il, s);
    return xlds ? launch_fold<WPL, NW, SEGR, D, VR, false, true>(x, qw, sc, qz, y, M, K, N, G, il, s)
                : launch_fold<WPL, NW, SEGR, D, VR, false, false>(x, qw, sc, qz, y, M, K, N, G, il, s);
}

template <int WPL, int NW, int SEGR, int D>
hipError_t launch_fold_m(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                         const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                         hipStream_t s) {
    switch (live_rows(M)) {
    case 1: return launch_fold_vr<WPL, NW, SEGR, D, 1>(x, qw, sc, qz, y, M, K, N, G, il, s);
    case 2: return launch_fold_vr<WPL, NW, SEGR, D, 2>(x, qw, sc, qz, y, M, K, N, G, il, s);
    default: return launch_fold_vr<WPL, NW, SEGR, D, 4>(x, qw, sc, qz, y, M, K, N, G, il, s);
    }
}

// Picks the wave count (a divisor of the segment count, at most 8) and the
// pipeline depth (the largest of 4, 2, 1 dividing the segments per wave).
template <int WPL, int SEGR>
hipError_t launch_fold_any(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                           const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                           hipStream_t s) {
    const int nseg = K / 8 / SEGR;
    if (nseg % 8 == 0) {
        const int per = nseg / 8;
        if (per % 4 == 0) return launch_fold_m<WPL, 8, SEGR, 4>(x, qw, sc, qz, y, M, K, N, G, il, s);
        if (per % 2 == 0) return launch_fold_m<WPL, 8, SEGR, 2>(x, qw, sc, qz, y, M, K, N, G, il, s);
        return launch_fold_m<WPL, 8, SEGR, 1>(x, qw, sc, qz, y, M, K, N, G, il, s);
    }
    if (nseg % 4 == 0) return launch_fold_m<WPL, 4, SEGR, 1>(x, qw, sc, qz, y, M, K, N, G, il, s);
    if (nseg % 2 == 0) return launch_fold_m<WPL, 2, SEGR, 1>(x, qw, sc, qz, y, M, K, N, G, il, s);
    return launch_fold_m<WPL, 1, SEGR, 1>(x, qw, sc, qz, y, M, K, N, G, il, s);
}

template <int WPL, int NW>
hipError_t launch_exact(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                        const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                        hipStream_t s) {
    constexpr int TN = 16 * WPL;
    hipLaunchKernelGGL((exact_kernel<WPL, NW>), dim3((N + TN - 1) / TN), dim3(NW * 64),
                       (size_t)NW * M * TN * sizeof(float), s, x,
                       reinterpret_cast<const uint32_t *>(qw), sc,
                       reinterpret_cast<const uint32_t *>(qz), y, M, K, N, G, il);
    return hipGetLastError();
}

// Fused gate/up: 8 words per lane (4 gate + 4 up columns), all live rows.  X
// staged segment by segment (prog), or in LDS before the loop (one row, where
// it fits).  The shape must fit stream_kernel.  Depth 1 throughout: on the 4096 x 28672
// [gate | up] layer, against depth 2 and X staged up front up to four rows,
// 1 row 13.07 -> 12.47 us, 2 rows 13.46 -> 12.05, 4 rows 16.28 -> 12.40,
// 8 rows 14.94 -> 12.81, 16 rows 16.03 -> 13.73-13.93.
template <int NW, int D, int IL>
hipError_t launch_gate_up(bool prog, const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                          const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                          hipStream_t s) {
    if (prog) return launch_stream_prog<8, NW, D, 1, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    const bool sym = qz == nullptr, grp1 = G == 8 * 16;
    const bool big = M * ((K / 128 + NW - 1) / NW) * 16 > 128;   // the largest wave's chunks
    if (M == 1) {   // one live C row per lane: 12.54 -> 12.23 us at one row
#define AWQ_GU1(SYMV, GRPV, XCHV) \
    launch_stream<8, NW, 16, D, 1, SYMV, GRPV, XCHV, true, 0, IL>(x, qw, sc, qz, y, M, K, N, G, s)
        if (big) {
            if (sym) return grp1 ? AWQ_GU1(true, true, kStageChunks) : AWQ_GU1(true, false, kStageChunks);
            return grp1 ? AWQ_GU1(false, true, kStageChunks) : AWQ_GU1(false, false, kStageChunks);
        }
        if (sym) return grp1 ? AWQ_GU1(true, true, 2) : AWQ_GU1(true, false, 2);
        return grp1 ? AWQ_GU1(false, true, 2) : AWQ_GU1(false, false, 2);
#undef AWQ_GU1
    }
#define AWQ_GU(SYMV, GRPV, XCHV) \
    launch_stream<8, NW, 16, D, 4, SYMV, GRPV, XCHV, true, 0, IL>(x, qw, sc, qz, y, M, K, N, G, s)
    if (big) {
        if (sym) return grp1 ? AWQ_GU(true, true, kStageChunks) : AWQ_GU(true, false, kStageChunks);
        return grp1 ? AWQ_GU(false, true, kStageChunks) : AWQ_GU(false, false, kStageChunks);
    }
    if (sym) return grp1 ? AWQ_GU(true, true, 2) : AWQ_GU(true, false, 2);
    return grp1 ? AWQ_GU(false, true, 2) : AWQ_GU(false, false, 2);
#undef AWQ_GU
}

// Fused gate/up launcher for one layout (awq_gemv_gate_up*.hip instantiate it).
template <int IL>
hipError_t gate_up_layout(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                                 const int32_t *qzeros, uint16_t *h, int M, int K, int N, int G,
                                 hipStream_t s) {
    // One row: X staged up front where it fits LDS.  Otherwise, and for more
    // rows, segment by segment, which takes any K.
    const bool up_front = M == 1 && stream_fits(M, K, N, G, 8, 8, 16, 1);
    if (!up_front && stream_fits_prog(M, K, N, G, 8, 8, 1))
        return launch_gate_up<8, 1, IL>(true, x, qweight, scales, qzeros, h, M, K, N, G, s);
    if (stream_fits(M, K, N, G, 8, 8, 16, 1))
        return launch_gate_up<8, 1, IL>(M > 1, x, qweight, scales, qzeros, h, M, K, N, G, s);
    if (stream_fits(M, K, N, G, 8, 2, 16, 1))
        return launch_gate_up<2, 1, IL>(M > 1, x, qweight, scales, qzeros, h, M, K, N, G, s);
    if (stream_fits(M, K, N, G, 8, 1, 16, 1))
        return launch_gate_up<1, 1, IL>(M > 1, x, qweight, scales, qzeros, h, M, K, N, G, s);
    return hipErrorNotSupported;
}

// One instantiated family of launchers per translation unit (arguments as
// launch_stream's): the staged kernel on canonical words (name), on interleaved
// ones (name_il) and on blocked ones (name_blk); the folded and exact kernels
// take the layout as an argument.
using Launcher = hipError_t(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                            const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                            hipStream_t s);
using LayoutLauncher = hipError_t(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                                  const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                                  int il, hipStream_t s);
Launcher gate_up, gate_up_il, gate_up_blk;
Launcher stream_m_w2_d2, stream_m_w2_d2_il, stream_m_w2_d2_blk;
Launcher stream_m_w4_d2, stream_m_w4_d2_il, stream_m_w4_d2_blk;
Launcher stream_m_w4_d1, stream_m_w4_d1_il, stream_m_w4_d1_blk;
Launcher prog_w2, prog_w2_il, prog_w2_blk;
Launcher prog_w4, prog_w4_il, prog_w4_blk;
Launcher prog_w8, prog_w8_il, prog_w8_blk;
LayoutLauncher fold_w2_s16;
LayoutLauncher fold_w4_s16;
LayoutLauncher fold_w4_s8;
LayoutLauncher fold_w4_s4;
LayoutLauncher exact_w4;

}  // namespace gemv
}  // namespace awq
