// Fused W4A16 dequantize-and-multiply for batches: AWQ's WQLinear_GEMM module,
// "GEMM for batch inference" (unfragile.ai AutoAWQ page, the WQLinear
// paragraph; pyshine.com AutoAWQ tour, overview bullets).  At M in the
// thousands this is a dense contraction, bound by the matrix cores.
//
// Workgroup: 256 threads = 4 waves, output tile BM x 256.  Wave w owns the 64
// columns [64 w, 64 w + 64) of the tile for all BM rows, so every packed
// weight is loaded and dequantized by exactly one wave, straight into the
// registers of an MFMA B operand (a packed word is 8 k of one column: one
// lane's B operand).  Dequantization is exact: w = fp16_rne(s (q - z)), the
// same bits awq_dequant writes; on one-group layers (G = K) the B operand is
// q - z and each column's scale multiplies its fp32 sums once, in the epilogue.
// X is the shared operand: each K step loads the
// BM x BK slice of X once per workgroup into LDS, XOR-swizzled per row, and all
// four waves read their A operands from there.
//
// Two kernels:
//   m32::mfma32_kernel (G a multiple of 32 and K of 128): v_mfma_f32_32x32x16,
//     a four-step ring of direct-to-LDS loads, 128- or 256-row tiles; also
//     the split-K mode (fp32 partial tiles per K slice, then
//     splitk_reduce_kernel adds the slices in order) and the fused gate/up
//     epilogue;
//   gemm_kernel (every other shape): v_mfma_f32_16x16x32, packed words loaded
//     into registers, clamped addresses and the weights of k past K zeroed.
//
// Tiles are assigned so that the workgroups one XCD runs (workgroup ids are
// dealt to the 8 XCDs round-robin) cover a compact block of output tiles:
// their X rows and weight columns then stay in that XCD's L2.
//
// This header holds the kernels and their layout-templated launchers;
// awq_gemm_canon.hip and awq_gemm_il.hip instantiate them once per word layout,
// awq_gemm.hip holds the entry points and the split-K reduction.
#pragma once
#include "awq_device.h"
#include "awq_timeline.h"
#include "awq_internal.h"

namespace awq {
namespace gemm {

constexpr int kBN = 256;      // tile columns (4 waves x 64)
constexpr int kBK = 64;       // k per step
constexpr int kXcds = 8;      // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kCus = kXcds * 32;

// 64-row tiles (MT 2) instead of 128-row ones: up to 64 rows, where a 128-row
// tile spends half its MFMAs or more on padding, and wherever 64-row tiles
// still fit one per CU, where they double the workgroups at work (4096 x 4096
// at 512 rows: 44.4 -> 38.5 us; 4096 x 28672 at 128 rows: 48.5 -> 42.0 us;
// beyond one tile per CU the 128-row tiles are faster).  Each output's sum
// runs over k in the same order either way: the results are bit-identical.
inline bool rows64(int M, int N) {
    return M <= 64 || (long long)((M + 63) / 64) * ((N + kBN - 1) / kBN) <= kCus;
}
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

// 4 bytes per lane from a buffer straight into LDS: lane i writes word i of dst.
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t rs, uint4 *dst,
                                               uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff, soff, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS: lane i writes dst + i.
__device__ __forceinline__ void global_to_lds16(const void *src, uint4 *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// General path, for the shapes the 32x32 kernels below do not take (G not a
// multiple of 32 or K not a multiple of 128): 16x16x32 MFMAs, packed words in
// registers, clamped addresses, and the weights of k past K zeroed.
// il: interleaved packed words, turned back to canonical order as they are read.
template <int BM, bool SYM>
__global__ void __launch_bounds__(256)
gemm_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ Q,
            const uint16_t *__restrict__ S, const uint32_t *__restrict__ QZ,
            uint16_t *__restrict__ Y, int M, int K, int N, int G, int il) {
    constexpr int MT = BM / 16;                    // 16-row MFMA tiles per wave
    constexpr int ACH = BM * kBK / 8 / 256;        // X chunks per thread per step
    constexpr int P = kRing - 1;                   // steps loaded ahead
    constexpr int BLOADS = SYM ? 4 : 6;
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
    const bool blk = il == 2;   // il: the qweight layout (nonzero: interleaved nibbles)
    const int qp = q_pitch(blk, N);
    const uint32_t qc = q_col(blk, ncl, KR);

    // X: chunk p of a tile (16 bytes) is written by lane p % 64 of one wave's
    // direct-to-LDS load; the swizzle is undone on the global side, so chunk p
    // holds (row p / 8, k chunk (p % 8) ^ (row & 7)).  Rows past M read row
    // M - 1 (their outputs are dropped).
    int xrow[ACH], xkc[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int p = (i * 4 + wave) * 64 + lane;
        const int row = p >> 3;
        xrow[i] = min(m0 + row, M - 1);
        xkc[i] = (p & 7) ^ (row & 7);
    }

    auto load_x = [&](int kt, uint4 *buf) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            uint4 *dst = buf + (i * 4 + wave) * 64;
            int gk = kt * kBK + xkc[i] * 8;
            gk = gk < K ? gk : 0;     // k past K: any valid address, weights are zeroed
            global_to_lds16(X + (size_t)xrow[i] * K + gk, dst);
        }
    };
    auto load_b = [&](int kt, BStep &b) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int r0 = kt * (kBK / 8) + 4 * s + kb;
            const int r = r0 < KR ? r0 : KR - 1;
            const int g = (8 * r) / G;
            b.q[s] = *reinterpret_cast<const uint4 *>(Q + (size_t)r * qp + qc);
            b.sc[s] = *reinterpret_cast<const uint2 *>(S + (size_t)g * N + ncl);
            if constexpr (SYM) b.zw[s] = 0x88888888u;
            else b.zw[s] = QZ[(size_t)g * (N / 8) + ncl / 8];
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
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            decode(cur.sc[s], cur.zw[s]);
            uint32_t q4[4] = {cur.q[s].x, cur.q[s].y, cur.q[s].z, cur.q[s].w};
            if (il)
#pragma unroll
                for (int i = 0; i < 4; ++i) q4[i] = deinterleave_word(q4[i]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t p[4], d[4];
                unpack_biased(q4[i], nmask, p);
#pragma unroll
                for (int j = 0; j < 4; ++j) d[j] = dequant_pair(p[j], bz2[i], s2[i]);
                uint4 w = pairs_to_natural(d);
                if (kt * (kBK / 8) + 4 * s + kb >= KR) w = make_uint4(0u, 0u, 0u, 0u);
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

// ---------------------------------------------------------------------------
// Fast path on 32x32x16 MFMAs: steps of BK = 64 k (G % 64 == 0, K % 256 == 0)
// or 32 k (G % 32 == 0, K % 128 == 0), 128- or 256-row tiles.
//
// A v_mfma_f32_32x32x16_f16 keeps the matrix core busy for 32 cycles, twice as
// long as the 16x16x32 form for the same operand registers, so one wave per
// SIMD can issue the whole dequantization of the next step's weights between
// its MFMAs without slowing them.  Wave w still owns the 64 columns
// [64 w, 64 w + 64) of the 128 x 256 tile, now as 4 row tiles x 2 column tiles
// of 32 x 32: the lane with column slot j (lane % 32) owns the adjacent columns
// 2 j and 2 j + 1 (column tiles 0 and 1), and half h = lane / 32 of the 16 k of
// an MFMA, i.e. packed row 2 kb + h of k block kb.
//
// Every load of the loop is a direct-to-LDS buffer load -- X, packed words,
// scales and zero points -- so all waits are the explicit counts below:
// the compiler tracks no vector-memory result in registers.  A step kt:
//   MFMAs of kt's k blocks but the last (B dequantized during kt - 1),
//   interleaved with the A reads of kt and the dequantization of kt + 1;
//   wait until X(kt + 1) and the weights of kt + 2 have landed, barrier;
//   issue the loads of step kt + 4 into the ring slots of kt;
//   read A(kt + 1, block 0) and the packed words of kt + 2 from LDS while the
//   last block's MFMAs run, and dequantize the last block of kt + 1.
// ---------------------------------------------------------------------------
namespace m32 {

// Geometry of one kernel variant: KB k blocks of 16 per step (BK = 16 KB k),
// MT row tiles of 32 per wave (BM = 32 MT rows per workgroup).
template <int KB, int MT>
struct Geom {
    static constexpr int BK = 16 * KB;
    static constexpr int BM = 32 * MT;
    static constexpr int XCH = BK / 8;               // 16-byte chunks per X row
    static constexpr int ACH = BM * XCH / 256;       // X chunks per thread per step
    static constexpr int QROWS = 2 * KB;             // packed rows per step
    static constexpr int QD = QROWS / 4;             // 16-byte packed-row loads per lane per step
    // Per-wave LDS region of one step's weights, in 16-byte chunks: QROWS
    // packed rows x 64 columns (row r, slot c at word 64 r + c), then 64 scale
    // words (word i: the scales of slots 2 (i % 32), +1), then 64 zero words
    // (word i: the zero word of slots 8 (i % 8) ..).
    static constexpr int SCALE = QROWS * 64 / 4;
    static constexpr int ZERO = SCALE + 16;
    static constexpr int WAVE = ZERO + 16;
};

// LDS chunk of (row, 16-byte k chunk kc) in an X tile of XCH chunks per row,
// XOR-swizzled so that the A-operand read of one k chunk by 16 consecutive
// rows (16 lanes of a 16-byte LDS read) falls in 16 different 16-byte bank
// groups of a 256-byte span, and the read by any 8 consecutive rows in 8
// different ones of a 128-byte span.  128-byte X rows (XCH 8): rows r and
// r + 8 share r & 7 and a 256-byte span's bank groups, so the XOR of r + 8
// differs in its low bit; 64-byte rows (XCH 4): the XOR (r / 2) ^ (r / 8)
// differs between the rows that share r % 2 in 8 and those that share r % 4
// in 16.
template <int XCH>
__device__ __forceinline__ int xswz(int row, int kc) {
    return row * XCH + (kc ^ (XCH == 8 ? ((row & 7) ^ ((row >> 3) & 1)) : (((row >> 1) ^ (row >> 3)) & 3)));
}

typedef float float16x_t __attribute__((ext_vector_type(16)));

// Natural-order unpack of one packed word: pair b = (k 2b, 2b+1) as the fp16
// pair (1024 + q_2b, 64 + q_2b+1).  v_perm copies byte b of the word into
// bytes 0 and 2 next to the exponent bytes 0x64 and 0x54; the mask keeps the
// low nibble in the low half (units at bit 0 of a 1024-based half) and the high
// nibble in the high half (units at bit 4 of a 64-based half).
__device__ __forceinline__ void unpack_natural(uint32_t w, uint32_t exps, uint32_t p[4]) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
        p[b] = __builtin_amdgcn_perm(exps, w, (7u << 24) | ((uint32_t)b << 16) | (5u << 8) | (uint32_t)b) &
               0xFFF0FF0Fu;
}

// GMODE, how step kt finds its group: 1, kt >> gshift (G / BK a power of
// two); 0, kt / (G / BK); 2, one group (G == K): each lane then loads its scale
// pair and zero word once, into registers, before the loop, and the steps load
// and decode only packed words.  B is then q - z, exact, and the column's scale
// multiplies the fp32 sums in the epilogue: one VALU fewer per weight pair, and
// no rounding of s (q - z) to fp16 (the output differs from x times
// awq_dequant's weights by that rounding, well inside the layer's tolerance).
// SPLIT (split K): workgroup row blockIdx.y sums only the k in slice
// [y kslice, (y + 1) kslice), which starts on a group boundary (or lies in the
// single group), and writes its fp32 partial tile to Y taken as float
// [slices][M][N]; a second kernel adds the slices.
// GU (fused gate/up): the layer's N = 2I columns are [gate | up].  A wave's 64
// MFMA columns are then 32 gate columns and the same 32 columns of the up half
// (column tile 0: gate, tile 1: up, for the same output column), and the
// output is h[M][I] = fp16(SiLU(gate) * up), 32 columns per wave.
// IL: the qweight layout (0 canonical, 1 interleaved, 2 blocked).  Nonzero:
// interleaved nibbles; each natural-order pair is then one AND-OR
// (unpack_interleaved), against the two v_perm + AND of the canonical word, and
// the bias of a pair is 1024 + z for the even pairs and 64 + z for the odd
// ones.  2: a wave's 64 columns lie in one 128-column block, whose packed rows
// are 512 bytes apart (q_col, q_pitch).
template <int KB, int MT, bool SYM, int GMODE, bool GU, bool SPLIT = false, int IL = 0>
__global__ void __launch_bounds__(256)
mfma32_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ Q,
              const uint16_t *__restrict__ S, const uint32_t *__restrict__ QZ,
              uint16_t *__restrict__ Y, int M, int K, int N, int G, int gshift, int kslice) {
    AWQ_TL_STAMP(tl_start);
    constexpr bool ONEG = GMODE == 2;
    static_assert(!(ONEG && GU), "one-group mode is for the plain layer");
    static_assert(!(SPLIT && GU), "split K is for the plain layer");
    using Gm = Geom<KB, MT>;
    constexpr int kBM = Gm::BM, kMT = MT, kACH = Gm::ACH, kWave = Gm::WAVE;
    constexpr int kScale = Gm::SCALE, kZero = Gm::ZERO, kBKs = Gm::BK, kXCH = Gm::XCH;
    constexpr int BLOADS = Gm::QD + (ONEG ? 0 : (SYM ? 1 : 2));   // per step: packed rows, scales, zeros
    constexpr int LOADS = kACH + BLOADS;
    __shared__ __attribute__((aligned(16))) uint4 ring0[kBM * kXCH];
    __shared__ __attribute__((aligned(16))) uint4 ring1[kBM * kXCH];
    __shared__ __attribute__((aligned(16))) uint4 ring2[kBM * kXCH];
    __shared__ __attribute__((aligned(16))) uint4 ring3[kBM * kXCH];
    __shared__ __attribute__((aligned(16))) uint4 bring0[4 * kWave];
    __shared__ __attribute__((aligned(16))) uint4 bring1[4 * kWave];
    __shared__ __attribute__((aligned(16))) uint4 bring2[4 * kWave];
    __shared__ __attribute__((aligned(16))) uint4 bring3[4 * kWave];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;
    const int h = lane >> 5;
    const int I = N / 2;                          // GU: output width
    const int tiles_m = (M + kBM - 1) / kBM;
    const int tiles_n = GU ? (I + kBN / 2 - 1) / (kBN / 2) : (N + kBN - 1) / kBN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kBM;
    const int n0 = tn * kBN + 64 * wave;          // first weight column of the wave
    const int hw0 = tn * (kBN / 2) + 32 * wave;   // GU: first output column of the wave
    // Layer column of slot c (0..63) of the wave's weight tile.
    auto src_col = [&](int c) { return GU ? (c < 32 ? hw0 + c : I + hw0 + c - 32) : n0 + c; };
    // The k this workgroup sums: all of K, or its slice under split K.
    const int k0 = SPLIT ? (int)blockIdx.y * kslice : 0;
    const int KL = SPLIT ? kslice : K;
    constexpr bool BLK = blocked_layout(IL);
    const int qp = q_pitch(BLK, N);
    const int groups = ONEG ? 1 : (K - k0) / G;   // scale rows from the slice's first group on
    if constexpr (SPLIT) {
        X += k0;
        Q += (size_t)(k0 / 8) * qp;
        if constexpr (!ONEG) {
            S += (size_t)(k0 / G) * N;
            if constexpr (!SYM) QZ += (size_t)(k0 / G) * (N / 8);
        }
    }
    const int KR = KL / 8;
    const int KT = KL / kBKs;

    // Buffer loads past a buffer's end return zeros; columns at or past N read
    // the next packed row (in bounds) and their outputs are dropped.  X rows
    // keep their stride K; the buffer ends after the slice's part of row M - 1.
    const __amdgpu_buffer_rsrc_t xrs =
        make_rsrc(X, ((uint32_t)(M - 1) * (uint32_t)K + (uint32_t)KL) * 2u);
    // Blocked words: the buffer runs to the end of qweight (every block's rows
    // of the slice lie in it; columns past N fall past its end and read zeros).
    const uint32_t qwords = BLK ? (uint32_t)(K / 8) * (uint32_t)N - (uint32_t)(k0 / 8) * kQBlock
                                : (uint32_t)KR * (uint32_t)N;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q, qwords * 4u);
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(S, (uint32_t)groups * (uint32_t)N * 2u);
    const __amdgpu_buffer_rsrc_t zrs = make_rsrc(QZ, SYM ? 0u : (uint32_t)groups * (uint32_t)N / 2u);
    uint32_t xvoff[kACH];
#pragma unroll
    for (int i = 0; i < kACH; ++i) {
        const int p = (i * 4 + wave) * 64 + lane;
        const int row = p / kXCH;
        const int xr = min(m0 + row, M - 1);
        const int xkc = (p % kXCH) ^ (xswz<kXCH>(row, 0) - row * kXCH);
        xvoff[i] = ((uint32_t)xr * (uint32_t)K + (uint32_t)xkc * 8u) * 2u;
    }
    // packed rows: load d (0, 1) of a step, lane i -> row 4 d + i / 16, columns n0 + 4 (i % 16) ..
    const uint32_t qvoff =
        ((uint32_t)(lane >> 4) * (uint32_t)qp + q_col(BLK, src_col(4 * (lane & 15)), K / 8)) * 4u;
    const uint32_t svoff = (uint32_t)src_col(2 * (lane & 31)) * 2u;
    const uint32_t zvoff = (uint32_t)(src_col(8 * (lane & 7)) / 8) * 4u;

    // Byte strides: a step of packed rows, half of it, a scale row, a zero row.
    const int qstep = Gm::QROWS * 4 * qp, qhalf = 16 * qp, srow = 2 * N, zrow = N / 2;
    const int gsteps = G / kBKs;
    auto load_step = [&](int kt, uint4 *xbuf, uint4 *bbuf) {
        uint4 *dst = bbuf + wave * kWave;
        const int qo = kt * qstep;
#pragma unroll
        for (int d = 0; d < Gm::QD; ++d) buffer_to_lds16(qrs, dst + 64 * d, qvoff, qo + d * qhalf);
        if constexpr (!ONEG) {
            const int g = GMODE == 1 ? (kt >> gshift) : kt / gsteps;
            buffer_to_lds4(srs, dst + kScale, svoff, g * srow);
            if constexpr (!SYM) buffer_to_lds4(zrs, dst + kZero, zvoff, g * zrow);
        }
#pragma unroll
        for (int i = 0; i < kACH; ++i)
            buffer_to_lds16(xrs, xbuf + (i * 4 + wave) * 64, xvoff[i], kt * kBKs * 2);
    };

    // Raw weights of one step for this lane: packed rows 2 kb + h, columns
    // n0 + 2 j, +1; the scale pair and the zero word of those columns.
    struct Raw {
        uint2 q[KB];
        uint32_t sc, zw;
    };
    // GU: slots j (gate) and 32 + j (up); sc = gate | up << 16, zw = the two
    // zero nibbles (gate in bits 0..3, up in 4..7).
    auto read_raw = [&](const uint4 *bbuf) {
        const uint32_t *w = reinterpret_cast<const uint32_t *>(bbuf + wave * kWave);
        Raw r;
        if constexpr (GU) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                r.q[kb] = make_uint2(w[64 * (2 * kb + h) + j], w[64 * (2 * kb + h) + 32 + j]);
            const uint32_t sg = w[4 * kScale + (j >> 1)] >> (16 * (j & 1));
            const uint32_t su = w[4 * kScale + 16 + (j >> 1)] >> (16 * (j & 1));
            r.sc = (sg & 0xFFFFu) | (su << 16);
            if constexpr (SYM) {
                r.zw = 0x88u;
            } else {
                const uint32_t zg = w[4 * kZero + (j >> 3)] >> (4 * (j & 7));
                const uint32_t zu = w[4 * kZero + 4 + (j >> 3)] >> (4 * (j & 7));
                r.zw = (zg & 0xFu) | ((zu & 0xFu) << 4);
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                r.q[kb] = *reinterpret_cast<const uint2 *>(w + 64 * (2 * kb + h) + 2 * j);
            if constexpr (ONEG) {
                r.sc = 0u;        // unused: the hoisted scales serve every step
                r.zw = 0u;
            } else {
                r.sc = w[4 * kScale + j];
                r.zw = SYM ? 0x88888888u : w[4 * kZero + (j >> 2)];
            }
        }
        return r;
    };
    const uint32_t exps = 0x54006400u;
    const uint32_t lo_mask = IL ? nibble_mask_vgpr() : 0u, hi_mask = IL ? high_mask_vgpr() : 0u;
    half8_t bA[KB][2], bB[KB][2];
    // Biased zero pairs and scale pairs of the two columns: (1024 + z, 64 + z)
    // for every canonical pair; for interleaved words (1024 + z, 1024 + z) for
    // the even pairs (bz2) and (64 + z, 64 + z) for the odd ones (bzo).
    struct Dq {
        half2_t bz2[2], bzo[2], s2[2];
    };
    auto decode = [&](const Raw &r) {
        Dq dq;
        const uint32_t z2 = GU ? r.zw : r.zw >> (8 * (j & 3));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const uint32_t z = (z2 >> (4 * ct)) & 0xFu;
            if constexpr (IL) {
                dq.bz2[ct] = as_half2(kBias1024x2 | (z << 16) | z);
                dq.bzo[ct] = as_half2(kBias64x2 | (z << 20) | (z << 4));
            } else {
                dq.bz2[ct] = as_half2(0x54006400u | (z << 20) | z);
                dq.bzo[ct] = dq.bz2[ct];
            }
            const half_t sv = as_half((uint16_t)(r.sc >> (16 * ct)));
            dq.s2[ct] = half2_t{sv, sv};
        }
        return dq;
    };

    float16x_t acc[kMT][2];
#pragma unroll
    for (int t = 0; t < kMT; ++t)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[t][ct][v] = 0.f;

    // A operands of k block kb of a step: row tiles t = 0 .. MT - 1.
    auto read_a = [&](const uint4 *xbuf, int kb, half8_t (&a)[kMT]) {
#pragma unroll
        for (int t = 0; t < kMT; ++t) a[t] = as_half8(xbuf[xswz<kXCH>(32 * t + j, 2 * kb + h)]);
    };
    auto mfma_kb = [&](const half8_t (&a)[kMT], const half8_t (&b)[2]) {
#pragma unroll
        for (int t = 0; t < kMT; ++t)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                acc[t][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[t], b[ct], acc[t][ct], 0, 0, 0);
    };
    auto dequant_kb = [&](const Raw &r, const Dq &dq, int kb, half8_t (&b)[2]) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            uint32_t p[4], d[4];
            if constexpr (IL) unpack_interleaved(ct ? r.q[kb].y : r.q[kb].x, lo_mask, hi_mask, p);
            else unpack_natural(ct ? r.q[kb].y : r.q[kb].x, exps, p);
            // One group: B is q - z (exact small integers); the column's scale
            // multiplies the fp32 sums once, in the epilogue.
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const half2_t bz = e % 2 ? dq.bzo[ct] : dq.bz2[ct];
                d[e] = ONEG ? as_u32(as_half2(p[e]) - bz) : dequant_pair(p[e], bz, dq.s2[ct]);
            }
            b[ct] = as_half8(make_uint4(d[0], d[1], d[2], d[3]));
        }
    };

    // Step kt, software-pipelined inside its MFMAs (KB k blocks x MT row tiles
    // x 2 column tiles).  On entry: b_cur = weights of kt (dequantized), a0 =
    // A(kt, kb 0), r = the packed weights of kt + 1 (read from LDS).  Each k
    // block's MFMAs run while the next block's A operands are read and one
    // block of step kt + 1's weights is dequantized.  Before the last block
    // the wave waits until everything up to step kt + 2 has landed (and its own
    // LDS reads of slot kt are done) and meets the other waves at a barrier.
    // After it, X(kt + 1) is visible to all waves, so the last block reads
    // A(kt + 1, kb 0) and the packed weights of kt + 2, and the loads of step
    // kt + 4 go into the ring slots of kt.  Neither LDS latency nor the
    // barrier reaches the matrix cores by more than a block's lead.
    // VALU slots between two MFMAs in the schedule.  With 64-k steps, 4 for
    // either layout: on interleaved words (about 3.3 dequantization VALU per
    // MFMA) 3 leaves a tail of VALU after the last MFMA before the barrier,
    // and 4 measured 1.6 to 3.4% faster (4096 x 4096, M 2048, K 4096 and
    // 16384); 5 and 6 are slower again.
    constexpr int VG = KB == 2 ? 2 : 4;
    half8_t a0[kMT], a1[kMT];
    Raw r;
    // One group: the lane's scale pair (columns n0 + 2 j, +1) and zero word,
    // loaded once; buffer loads past the end (columns at or past N) give 0.
    Dq dq_one{};
    if constexpr (ONEG) {
        Raw hr{};
        hr.sc = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(srs, svoff, 0, 0);
        hr.zw = SYM ? 0x88888888u
                    : (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                          zrs, (uint32_t)((n0 >> 3) + (j >> 2)) * 4u, 0, 0);
        dq_one = decode(hr);
    }
    auto step = [&](int kt, const uint4 *xcur, half8_t (&b_cur)[KB][2], half8_t (&b_nxt)[KB][2],
                    const uint4 *xnxt, const uint4 *bnn, uint4 *xload, uint4 *bload) {
        __builtin_amdgcn_sched_barrier(0);
        const Raw rc = r;
        const Dq dq = ONEG ? dq_one : decode(rc);
        read_a(xcur, 1, a1);
#pragma unroll
        for (int kb = 0; kb < KB - 1; ++kb) {
            dequant_kb(rc, dq, kb, b_nxt[kb]);
            mfma_kb(kb % 2 ? a1 : a0, b_cur[kb]);
            if (kb + 2 < KB) read_a(xcur, kb + 2, kb % 2 ? a1 : a0);
        }
#pragma unroll
        for (int i = 0; i < (KB - 1) * kMT * 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, VG, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are done
        wait_vmcnt<LOADS>();                  // every batch but the last (step kt + 3) is in
        barrier_no_fence();
        __builtin_amdgcn_sched_barrier(0);
        load_step(min(kt + kRing, KT - 1), xload, bload);
        read_a(xnxt, 0, a0);
        r = read_raw(bnn);
        mfma_kb(a1, b_cur[KB - 1]);            // KB is even: the last block's A is in a1
        dequant_kb(rc, dq, KB - 1, b_nxt[KB - 1]);
#pragma unroll
        for (int i = 0; i < kMT * 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, VG, 0);  // VALU
        }
    };

    // Prologue: steps 0 .. 3 in flight; step 0 needs steps 0 and 1 landed.
    load_step(0, ring0, bring0);
    __builtin_amdgcn_sched_barrier(0);
    load_step(min(1, KT - 1), ring1, bring1);
    __builtin_amdgcn_sched_barrier(0);
    load_step(min(2, KT - 1), ring2, bring2);
    __builtin_amdgcn_sched_barrier(0);
    load_step(min(3, KT - 1), ring3, bring3);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2 * LOADS>();
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
    r = read_raw(bring0);
    {
        const Dq dq = ONEG ? dq_one : decode(r);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) dequant_kb(r, dq, kb, bA[kb]);
    }
    r = read_raw(bring1);
    read_a(ring0, 0, a0);
    AWQ_TL_STAMP(tl_loop0);
    AWQ_TL_CLOCK(tc_loop0);
    for (int kt = 0; kt < KT; kt += kRing) {
        step(kt + 0, ring0, bA, bB, ring1, bring2, ring0, bring0);
        step(kt + 1, ring1, bB, bA, ring2, bring3, ring1, bring1);
        step(kt + 2, ring2, bA, bB, ring3, bring0, ring2, bring2);
        step(kt + 3, ring3, bB, bA, ring0, bring1, ring3, bring3);
    }
    wait_vmcnt<0>();   // no load into LDS may outlive the workgroup
    AWQ_TL_STAMP(tl_loop1);
    AWQ_TL_CLOCK(tc_loop1);

    // C layout of the 32x32 MFMA: lane (h, j) holds, in register v, row
    // 8 (v / 4) + 4 h + v % 4 of column slot j.
    if constexpr (GU) {
        // column tiles 0 and 1 are gate and up of output column hw0 + j
        const int col = hw0 + j;
        if (col >= I) return;
#pragma unroll
        for (int t = 0; t < kMT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + 32 * t + 8 * (v / 4) + 4 * h + (v % 4);
                if (row < M) {
                    const float g = acc[t][0][v];
                    __builtin_nontemporal_store(as_u16((half_t)(g / (1.0f + __expf(-g)) * acc[t][1][v])),
                                                Y + (size_t)row * I + col);
                }
            }
        return;
    }
    // column tiles 0 and 1 are the adjacent columns n0 + 2 j and n0 + 2 j + 1,
    // stored as one 4-byte word (split K: one 8-byte fp32 pair of the slice's
    // partial tile).  The fp16 outputs (here and in the gate/up epilogue) are
    // nontemporal stores: every CU writes its whole tile at once at the end,
    // and lines that bypass the L2 need no write-back when the kernel ends
    // (prefill shape 61.3 -> 60.1 us; the waves' own time is unchanged).
    const int col = n0 + 2 * j;
    if (col >= N) return;
    if constexpr (ONEG) {
        const float s0 = (float)dq_one.s2[0][0], s1 = (float)dq_one.s2[1][0];
#pragma unroll
        for (int t = 0; t < kMT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc[t][0][v] *= s0;
                acc[t][1][v] *= s1;
            }
    }
    if constexpr (SPLIT) {
        float *Yf = reinterpret_cast<float *>(Y) + (size_t)blockIdx.y * M * N;
#pragma unroll
        for (int t = 0; t < kMT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + 32 * t + 8 * (v / 4) + 4 * h + (v % 4);
                if (row < M)
                    *reinterpret_cast<float2 *>(Yf + (size_t)row * N + col) =
                        make_float2(acc[t][0][v], acc[t][1][v]);
            }
        return;
    }
#pragma unroll
    for (int t = 0; t < kMT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = m0 + 32 * t + 8 * (v / 4) + 4 * h + (v % 4);
            if (row < M) {
                const uint32_t w = (uint32_t)as_u16((half_t)acc[t][0][v]) |
                                   ((uint32_t)as_u16((half_t)acc[t][1][v]) << 16);
                __builtin_nontemporal_store(w, reinterpret_cast<uint32_t *>(Y + (size_t)row * N + col));
            }
        }
#ifdef AWQ_TIMELINE
    __builtin_amdgcn_s_waitcnt(0);   // the stores have completed
    AWQ_TL_STAMP(tl_end);
    if (threadIdx.x == 0)
        awq_tl_record((int)(blockIdx.x + gridDim.x * blockIdx.y), tl_start, tl_loop0, tl_loop1, tl_end,
                      tc_loop0, tc_loop1);
#endif
}

template <int KB, int MT, bool SYM, bool GU, int IL>
hipError_t launch(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                  uint16_t *y, int M, int K, int N, int G, hipStream_t s) {
    using Gm = Geom<KB, MT>;
    const int tn = GU ? (N / 2 + kBN / 2 - 1) / (kBN / 2) : (N + kBN - 1) / kBN;
    const long long tiles = (long long)((M + Gm::BM - 1) / Gm::BM) * tn;
    const int gsteps = G / Gm::BK;
    int gshift = -1;
    if (G == K) gshift = 31;
    else if ((gsteps & (gsteps - 1)) == 0) gshift = __builtin_ctz((unsigned)gsteps);
    const auto *q = reinterpret_cast<const uint32_t *>(qw);
    const auto *z = reinterpret_cast<const uint32_t *>(qz);
    if constexpr (!GU) {
        if (G == K) {
            hipLaunchKernelGGL((mfma32_kernel<KB, MT, SYM, 2, false, false, IL>), dim3((unsigned)tiles), dim3(256),
                               0, s, x, q, sc, z, y, M, K, N, G, 0, K);
            return hipGetLastError();
        }
    }
    if (gshift >= 0)
        hipLaunchKernelGGL((mfma32_kernel<KB, MT, SYM, 1, GU, false, IL>), dim3((unsigned)tiles), dim3(256), 0,
                           s, x, q, sc, z, y, M, K, N, G, gshift, K);
    else
        hipLaunchKernelGGL((mfma32_kernel<KB, MT, SYM, 0, GU, false, IL>), dim3((unsigned)tiles), dim3(256), 0,
                           s, x, q, sc, z, y, M, K, N, G, 0, K);
    return hipGetLastError();
}

// Split K: `splits` slices of K / splits k, each a whole number of steps and
// of groups (or inside the single group), as a second grid dimension; fp32
// partial tiles into part[splits][M][N].
template <int KB, int MT, bool SYM, int IL>
hipError_t launch_split(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                        float *part, int M, int K, int N, int G, int splits, hipStream_t s) {
    using Gm = Geom<KB, MT>;
    const int kslice = K / splits;
    const long long tiles = (long long)((M + Gm::BM - 1) / Gm::BM) * ((N + kBN - 1) / kBN);
    const dim3 grid((unsigned)tiles, (unsigned)splits);
    const auto *q = reinterpret_cast<const uint32_t *>(qw);
    const auto *z = reinterpret_cast<const uint32_t *>(qz);
    auto *y = reinterpret_cast<uint16_t *>(part);
    const int gsteps = G / Gm::BK;
    if (G == K)
        hipLaunchKernelGGL((mfma32_kernel<KB, MT, SYM, 2, false, true, IL>), grid, dim3(256), 0, s, x, q, sc,
                           z, y, M, K, N, G, 0, kslice);
    else if ((gsteps & (gsteps - 1)) == 0)
        hipLaunchKernelGGL((mfma32_kernel<KB, MT, SYM, 1, false, true, IL>), grid, dim3(256), 0, s, x, q, sc,
                           z, y, M, K, N, G, __builtin_ctz((unsigned)gsteps), kslice);
    else
        hipLaunchKernelGGL((mfma32_kernel<KB, MT, SYM, 0, false, true, IL>), grid, dim3(256), 0, s, x, q, sc,
                           z, y, M, K, N, G, 0, kslice);
    return hipGetLastError();
}

}  // namespace m32

// Step size of the split-K kernel for slices of kslice k: 64 (or 32) k steps,
// whole ring turns, and whole groups unless there is a single group.
inline int splitk_bk(int K, int G, int splits) {
    if (splits < 1 || K % splits) return 0;
    const int kslice = K / splits;
    const bool groups_ok = G == K || kslice % G == 0;
    if (!groups_ok) return 0;
    if ((G == K || G % 64 == 0) && kslice % (kRing * 64) == 0) return 64;
    if ((G == K || G % 32 == 0) && kslice % (kRing * 32) == 0) return 32;
    return 0;
}

// The general kernel (16x16x32 MFMAs, any G and K), both layouts: it reads the
// layout as a kernel argument.
hipError_t launch_general(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                          const int32_t *qz, uint16_t *y, int M, int K, int N, int G, int il,
                          hipStream_t s);

// One layout's launchers, defined in awq_gemm_canon.hip (canonical words) and
// awq_gemm_il.hip (interleaved words).
using PlainLauncher = hipError_t(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                                 const int32_t *qz, uint16_t *y, int M, int K, int N, int G,
                                 hipStream_t s);
using SplitLauncher = hipError_t(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                                 const int32_t *qz, float *part, int M, int K, int N, int G,
                                 int splits, hipStream_t s);
PlainLauncher plain_canon, plain_il, plain_blk, gate_up_canon, gate_up_il, gate_up_blk;
SplitLauncher split_canon, split_il, split_blk;

// Kernel choice: 256-row tiles with 32-k steps for large batches (half the
// dequantization per MFMA), as long as they fill the GPU twice over; 128-row
// tiles with 64-k steps otherwise, 64-row ones where rows64 says; 32-k steps
// when G or K only allow those; the general kernel for the rest.
template <int IL>
hipError_t launch_layout(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                         uint16_t *y, int M, int K, int N, int G, hipStream_t s) {
    const bool sym = qz == nullptr;
    const bool k32 = G % 32 == 0 && K % (kRing * 32) == 0;
    const bool k64 = G % 64 == 0 && K % (kRing * 64) == 0;
    const long long wide_tiles = (long long)((M + 255) / 256) * ((N + kBN - 1) / kBN);
    if (k32 && wide_tiles >= 512)
        return sym ? m32::launch<2, 8, true, false, IL>(x, qw, sc, qz, y, M, K, N, G, s)
                   : m32::launch<2, 8, false, false, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    const bool small = rows64(M, N);
    if (k64 && small)
        return sym ? m32::launch<4, 2, true, false, IL>(x, qw, sc, qz, y, M, K, N, G, s)
                   : m32::launch<4, 2, false, false, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    if (k64)
        return sym ? m32::launch<4, 4, true, false, IL>(x, qw, sc, qz, y, M, K, N, G, s)
                   : m32::launch<4, 4, false, false, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    if (k32 && small)
        return sym ? m32::launch<2, 2, true, false, IL>(x, qw, sc, qz, y, M, K, N, G, s)
                   : m32::launch<2, 2, false, false, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    if (k32)
        return sym ? m32::launch<2, 4, true, false, IL>(x, qw, sc, qz, y, M, K, N, G, s)
                   : m32::launch<2, 4, false, false, IL>(x, qw, sc, qz, y, M, K, N, G, s);
    return launch_general(x, qw, sc, qz, y, M, K, N, G, IL, s);
}

// Split-K partial tiles: 64-k steps where splitk_bk allows them, else 32-k;
// 64-row tiles up to 64 rows (a 128-row tile would spend half its MFMAs or
// more on padding rows), and wherever the 64-row tiles times the slices still
// fit one workgroup per CU (4096 x 4096 at 128 rows in 8 slices: 22.4 -> 21.0
// us; at 256 rows in 4: 23.8 -> 22.1 us).
template <int IL>
hipError_t split_layout(const uint16_t *x, const int32_t *qw, const uint16_t *sc, const int32_t *qz,
                        float *part, int M, int K, int N, int G, int splits, hipStream_t s) {
    const bool sym = qz == nullptr;
    const bool r64 = M <= 64 || (long long)((M + 63) / 64) * ((N + kBN - 1) / kBN) * splits <= kCus;
#define AWQ_SPLIT(KBV, MTV)                                                                         \
    (sym ? m32::launch_split<KBV, MTV, true, IL>(x, qw, sc, qz, part, M, K, N, G, splits, s)        \
         : m32::launch_split<KBV, MTV, false, IL>(x, qw, sc, qz, part, M, K, N, G, splits, s))
    if (splitk_bk(K, G, splits) == 64) return r64 ? AWQ_SPLIT(4, 2) : AWQ_SPLIT(4, 4);
    return r64 ? AWQ_SPLIT(2, 2) : AWQ_SPLIT(2, 4);
#undef AWQ_SPLIT
}

// Fused gate/up: 64-row tiles where they pay, as in the plain GEMM (the tile
// count is the same: 128 output columns are 256 layer columns).
template <int IL>
hipError_t gate_up_layout(const uint16_t *x, const int32_t *qw, const uint16_t *sc,
                          const int32_t *qz, uint16_t *h, int M, int K, int N, int G,
                          hipStream_t s) {
    const bool r64 = rows64(M, N), sym = qz == nullptr;
    if (r64)
        return sym ? m32::launch<4, 2, true, true, IL>(x, qw, sc, qz, h, M, K, N, G, s)
                   : m32::launch<4, 2, false, true, IL>(x, qw, sc, qz, h, M, K, N, G, s);
    return sym ? m32::launch<4, 4, true, true, IL>(x, qw, sc, qz, h, M, K, N, G, s)
               : m32::launch<4, 4, false, true, IL>(x, qw, sc, qz, h, M, K, N, G, s);
}

}  // namespace gemm
}  // namespace awq
