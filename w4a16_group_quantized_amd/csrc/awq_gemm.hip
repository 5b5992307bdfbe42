// Fused W4A16 dequantize-and-multiply for batches: AWQ's WQLinear_GEMM module,
// "GEMM for batch inference" (unfragile.ai AutoAWQ page, the WQLinear
// paragraph; pyshine.com AutoAWQ tour, overview bullets).  At M in the
// thousands this is a dense contraction, bound by the matrix cores.
//
// Workgroup: 256 threads = 4 waves, output tile BM x 256.  Wave w owns the 64
// columns [64 w, 64 w + 64) of the tile for all BM rows, so every packed
// weight is loaded and dequantized by exactly one wave, straight into
// registers: one 16-byte load of a packed row gives a lane four words (four
// consecutive columns, 8 k each), and each word, dequantized, is that lane's B
// operand of one v_mfma_f32_16x16x32_f16 (8 k of one column).  The four words
// feed four MFMA column sets {4 c + i}.  Dequantization is exact:
// w = fp16_rne(s (q - z)), the same bits awq_dequant writes.
//
// X is the shared operand: each K step of BK = 64 loads the BM x 64 slice of X
// once per workgroup into LDS (16-byte chunks, each reordered to the (j, j+4)
// k pairing of the unpacked words, XOR-swizzled per row so that the 16 rows an
// A-operand read touches fall in different banks), and all four waves read
// their A operands from there.  The next step's X and packed words
// are loaded while the current step multiplies (double-buffered LDS).
//
// Tiles are assigned so that the workgroups one XCD runs (workgroup ids are
// dealt to the 8 XCDs round-robin) cover a compact block of output tiles:
// their X rows and weight columns then stay in that XCD's L2.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {
namespace gemm {

constexpr int kBN = 256;      // tile columns (4 waves x 64)
constexpr int kBK = 64;       // k per step
constexpr int kXcds = 8;      // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kGroupM = 4;    // tile rows per band of the tile order

// Workgroup id -> output tile (tm, tn).  Ids are dealt to XCDs round-robin, so
// id -> (xcd, slot); each XCD takes a contiguous range of the tile order, which
// walks bands of kGroupM tile rows column by column.
__device__ __forceinline__ void tile_of(int id, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int T = tiles_m * tiles_n;
    const int xcd = id % kXcds, slot = id / kXcds;
    const int base = T / kXcds, extra = T % kXcds;
    const int t = xcd * base + min(xcd, extra) + slot;
    const int band = t / (kGroupM * tiles_n);
    const int rows = min(kGroupM, tiles_m - band * kGroupM);
    const int in = t - band * kGroupM * tiles_n;
    tm = band * kGroupM + in % rows;
    tn = in / rows;
}

// LDS chunk index of (row, 16-byte k chunk kc) in a tile of 8 chunks per row.
__device__ __forceinline__ int swz(int row, int kc) { return row * 8 + (kc ^ (row & 7)); }

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// The packed words of one K step for one lane: rows 8 kt + 4 s + kb (s = 0, 1),
// four consecutive columns, with their scales and zero points.
struct BStep {
    uint4 q[2];
    uint2 sc[2];
    uint32_t zw[2];
};

// Workgroup barrier without the memory fence of __syncthreads (which would wait
// for every outstanding load, including the ones prefetching later steps).
// LDS data written by direct-to-LDS loads is covered by the explicit vmcnt wait
// that precedes it; the memory clobber keeps the compiler from moving LDS reads
// above it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// Four LDS ring buffers as separate objects, so that the compiler can tell an
// LDS read of one buffer from a direct-to-LDS load into another and need not
// wait for the latter.
constexpr int kRing = 4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane i writes dst + i.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rs, uint4 *dst,
                                                uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS: lane i writes dst + i.
__device__ __forceinline__ void global_to_lds16(const void *src, uint4 *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// FAST: G % 64 == 0 and K % (4 * 64) == 0 -- every step lies in one group and
// the steps fill whole rings, so all loads are buffer loads with a per-lane
// offset fixed for the kernel and a per-step offset in a scalar register (no
// address arithmetic in the loop), scales and zero points are decoded once per
// step, and no step needs masking.  Other shapes take the general path, which
// clamps addresses and zeroes the weights of k past K.
template <int BM, bool SYM, bool FAST>
__global__ void __launch_bounds__(256)
gemm_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ Q,
            const uint16_t *__restrict__ S, const uint32_t *__restrict__ QZ,
            uint16_t *__restrict__ Y, int M, int K, int N, int G) {
    constexpr int MT = BM / 16;                    // 16-row MFMA tiles per wave
    constexpr int ACH = BM * kBK / 8 / 256;        // X chunks per thread per step
    constexpr int P = kRing - 1;                   // steps loaded ahead
    constexpr int BLOADS = FAST ? (SYM ? 3 : 4) : (SYM ? 4 : 6);
    constexpr int LOADS = ACH + BLOADS;            // vector-memory loads per step per thread
    __shared__ __attribute__((aligned(16))) uint4 ring0[BM * 8];
    __shared__ __attribute__((aligned(16))) uint4 ring1[BM * 8];
    __shared__ __attribute__((aligned(16))) uint4 ring2[BM * 8];
    __shared__ __attribute__((aligned(16))) uint4 ring3[BM * 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15;
    const int kb = lane >> 4;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + kBN - 1) / kBN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * kBN + 64 * wave;           // this wave's first column
    const int ncol = n0 + 4 * c16;                 // this lane's 4 columns
    const bool col_ok = ncol < N;
    const int ncl = col_ok ? ncol : N - 4;         // clamped load column
    const int KR = K / 8;
    const int KT = (K + kBK - 1) / kBK;
    const int KTP = (KT + kRing - 1) / kRing * kRing;   // steps, padded to whole rings
    const uint32_t nmask = nibble_mask_vgpr();

    // X: chunk p of a tile (16 bytes) is written by lane p % 64 of one wave's
    // direct-to-LDS load; the swizzle is undone on the global side, so chunk p
    // holds (row p / 8, k chunk (p % 8) ^ (row & 7)).  Rows past M read row
    // M - 1 (their outputs are dropped).
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q, (uint32_t)KR * (uint32_t)N * 4u);
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(S, (uint32_t)(K / G) * (uint32_t)N * 2u);
    const __amdgpu_buffer_rsrc_t zrs = make_rsrc(QZ, SYM ? 0u : (uint32_t)(K / G) * (uint32_t)N / 2u);
    int xrow[ACH], xkc[ACH];
    uint32_t xvoff[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int p = (i * 4 + wave) * 64 + lane;
        const int row = p >> 3;
        xrow[i] = min(m0 + row, M - 1);
        xkc[i] = (p & 7) ^ (row & 7);
        xvoff[i] = ((uint32_t)xrow[i] * (uint32_t)K + (uint32_t)xkc[i] * 8u) * 2u;
    }
    const uint32_t qvoff = ((uint32_t)kb * (uint32_t)N + (uint32_t)ncl) * 4u;
    const uint32_t svoff = (uint32_t)ncl * 2u;
    const uint32_t zvoff = (uint32_t)(ncl / 8) * 4u;

    auto load_x = [&](int kt, uint4 *buf) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            uint4 *dst = buf + (i * 4 + wave) * 64;
            if constexpr (FAST) {
                buffer_to_lds16(xrs, dst, xvoff[i], kt * kBK * 2);
            } else {
                int gk = kt * kBK + xkc[i] * 8;
                gk = gk < K ? gk : 0;     // k past K: any valid address, weights are zeroed
                global_to_lds16(X + (size_t)xrow[i] * K + gk, dst);
            }
        }
    };
    auto load_b = [&](int kt, BStep &b) {
        if constexpr (FAST) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                    qrs, qvoff, (kt * (kBK / 8) + 4 * s) * N * 4, 0);
                b.q[s] = make_uint4(v.x, v.y, v.z, v.w);
            }
            const int g = (kt * kBK) / G;
            const u32x2 sv = __builtin_amdgcn_raw_buffer_load_b64(srs, svoff, g * N * 2, 0);
            b.sc[0] = make_uint2(sv.x, sv.y);
            if constexpr (SYM) b.zw[0] = 0x88888888u;
            else b.zw[0] = __builtin_amdgcn_raw_buffer_load_b32(zrs, zvoff, g * (N / 8) * 4, 0);
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int r0 = kt * (kBK / 8) + 4 * s + kb;
                const int r = r0 < KR ? r0 : KR - 1;
                const int g = (8 * r) / G;
                b.q[s] = *reinterpret_cast<const uint4 *>(Q + (size_t)r * N + ncl);
                b.sc[s] = *reinterpret_cast<const uint2 *>(S + (size_t)g * N + ncl);
                if constexpr (SYM) b.zw[s] = 0x88888888u;
                else b.zw[s] = QZ[(size_t)g * (N / 8) + ncl / 8];
            }
        }
    };

    float4_t acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = float4_t{0.f, 0.f, 0.f, 0.f};

    BStep bq[kRing];
    // One step: wait for its loads (issued P steps earlier; P - 1 later steps
    // may still be in flight), barrier (every wave's X tile is in LDS and every
    // wave is done reading the buffer reloaded next), issue step kt + P, then
    // dequantize and multiply step kt.
    auto step = [&](int kt, uint4 *cur_buf, BStep &cur, uint4 *next_buf, BStep &next) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(P - 1) * LOADS>();
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
        half8_t b[2][4];
        half2_t bz2[4], s2[4];
        auto decode = [&](const uint2 sc, uint32_t zw) {
            const uint32_t z4 = zw >> (4 * (ncl % 8));
            const uint16_t s4[4] = {(uint16_t)sc.x, (uint16_t)(sc.x >> 16), (uint16_t)sc.y,
                                    (uint16_t)(sc.y >> 16)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half_t bz = biased_zero(z4 >> (4 * i));
                const half_t sv = as_half(s4[i]);
                bz2[i] = half2_t{bz, bz};
                s2[i] = half2_t{sv, sv};
            }
        };
        if constexpr (FAST) decode(cur.sc[0], cur.zw[0]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if constexpr (!FAST) decode(cur.sc[s], cur.zw[s]);
            const uint32_t q4[4] = {cur.q[s].x, cur.q[s].y, cur.q[s].z, cur.q[s].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t p[4], d[4];
                unpack_biased(q4[i], nmask, p);
#pragma unroll
                for (int j = 0; j < 4; ++j) d[j] = dequant_pair(p[j], bz2[i], s2[i]);
                uint4 w = pairs_to_natural(d);
                if constexpr (!FAST) {
                    if (kt * (kBK / 8) + 4 * s + kb >= KR) w = make_uint4(0u, 0u, 0u, 0u);
                }
                b[s][i] = as_half8(w);
            }
        }
        {
            const int kn = min(kt + P, KT - 1);
            load_x(kn, next_buf);
            load_b(kn, next);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                // A operand: row 16 t + c16, k chunk 4 s + kb, natural k order.
                const half8_t a = as_half8(cur_buf[swz(16 * t + c16, 4 * s + kb)]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[s][i], acc[t][i], 0, 0, 0);
            }
        }
    };

    // Prologue: steps 0 .. P-1 in flight.
    load_x(0, ring0);
    load_b(0, bq[0]);
    load_x(min(1, KT - 1), ring1);
    load_b(min(1, KT - 1), bq[1]);
    load_x(min(2, KT - 1), ring2);
    load_b(min(2, KT - 1), bq[2]);
    for (int kt = 0; kt < KTP; kt += kRing) {
        step(kt + 0, ring0, bq[0], ring3, bq[3]);
        step(kt + 1, ring1, bq[1], ring0, bq[0]);
        step(kt + 2, ring2, bq[2], ring1, bq[1]);
        step(kt + 3, ring3, bq[3], ring2, bq[2]);
    }

    // C layout of the 16x16 MFMA: lane (kb, c16) of column set i holds rows
    // 4 kb + v of column 4 c16 + i: four consecutive columns per row.
    if (!col_ok) return;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = m0 + 16 * t + 4 * kb + v;
            if (row < M) {
                const uint32_t lo = (uint32_t)as_u16((half_t)acc[t][0][v]) |
                                    ((uint32_t)as_u16((half_t)acc[t][1][v]) << 16);
                const uint32_t hi = (uint32_t)as_u16((half_t)acc[t][2][v]) |
                                    ((uint32_t)as_u16((half_t)acc[t][3][v]) << 16);
                *reinterpret_cast<uint2 *>(Y + (size_t)row * N + ncol) = make_uint2(lo, hi);
            }
        }
}

template <int BM, bool SYM, bool FAST>
hipError_t launch_sym(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                      uint16_t *y, int M, int K, int N, int G, hipStream_t s) {
    const long long tiles = (long long)((M + BM - 1) / BM) * ((N + kBN - 1) / kBN);
    hipLaunchKernelGGL((gemm_kernel<BM, SYM, FAST>), dim3((unsigned)tiles), dim3(256), 0, s, x,
                       reinterpret_cast<const uint32_t *>(qw), sc,
                       reinterpret_cast<const uint32_t *>(qz), y, M, K, N, G);
    return hipGetLastError();
}

template <int BM>
hipError_t launch(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                  uint16_t *y, int M, int K, int N, int G, hipStream_t s) {
    const bool fast = G % kBK == 0 && K % (kRing * kBK) == 0;
    if (qz == nullptr)
        return fast ? launch_sym<BM, true, true>(x, qw, sc, qz, y, M, K, N, G, s)
                    : launch_sym<BM, true, false>(x, qw, sc, qz, y, M, K, N, G, s);
    return fast ? launch_sym<BM, false, true>(x, qw, sc, qz, y, M, K, N, G, s)
                : launch_sym<BM, false, false>(x, qw, sc, qz, y, M, K, N, G, s);
}

}  // namespace gemm

hipError_t launch_gemm(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                       const int32_t *qzeros, uint16_t *y, int M, int K, int N, int G,
                       hipStream_t s) {
    return gemm::launch<128>(x, qweight, scales, qzeros, y, M, K, N, G, s);
}

}  // namespace awq
