// Device-side building blocks shared by the HIP kernels of libawq (gfx950).
//
// Packed layout (see include/awq.h): a 32-bit qweight word holds the codes of
// eight consecutive k of one column, code j in bits 4j..4j+3; a qzeros word
// holds the zero points of eight consecutive columns of one group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

// fp16 whose bit pattern is 0x6400 | c has exponent 2^10 and ulp 1, so it is
// exactly 1024 + c for any 4-bit c.  This turns nibbles into halves with one
// AND-OR per two codes, no conversion instruction.
constexpr uint32_t kBias1024x2 = 0x64006400u;
constexpr uint32_t kNibblePairMask = 0x000F000Fu;

// The nibble-pair mask in a vector register that the optimizer cannot see
// through.  gfx9 VOP3 encodings take no literal constants and read at most one
// scalar register, so with both constants visible the compiler splits
// (x & mask) | bias into two literal-carrying VOP2 instructions; with the mask
// in a vector register it emits a single v_and_or_b32 (bias in a scalar
// register).  Call once per kernel, outside the loops.
__device__ __forceinline__ uint32_t nibble_mask_vgpr() {
    uint32_t v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(kNibblePairMask));
    return v;
}

// Splits a qweight word into four half2 registers
//   p[j] = (1024 + q_j, 1024 + q_{j+4}),  j = 0..3,
// with three shifts and four AND-ORs.  The pairing (j, j+4) is the one the
// shift-and-mask yields for free; callers feed the other operand in the same
// k order.  `mask` is kNibblePairMask (see nibble_mask_vgpr).
__device__ __forceinline__ void unpack_biased(uint32_t w, uint32_t mask, uint32_t p[4]) {
    p[0] = (w & mask) | kBias1024x2;
    p[1] = ((w >> 4) & mask) | kBias1024x2;
    p[2] = ((w >> 8) & mask) | kBias1024x2;
    p[3] = ((w >> 12) & mask) | kBias1024x2;
}

// All-reduce over aligned groups of L lanes (L = 2, 4, 8 or 16) with DPP lane
// moves, which stay in the vector ALU (a __shfl_xor is an LDS permute with its
// latency).  Step s combines each lane with a partner in the other half of its
// group of 2^(s+1) lanes: xor 1 and xor 2 within a quad, then the mirror lane
// within 8 and within 16.  After the steps before it the value is uniform
// within each half, so a mirror partner serves as well as an xor partner.
// op(a, b) must be commutative and associative (exactly, for the result to be
// the same in every lane: min and max are; a float sum is the same in every
// lane of the group but depends on the step order).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int L, typename Op>
__device__ __forceinline__ uint32_t lane_group_reduce(uint32_t v, Op op) {
    static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16, "group of 1..16 lanes");
    if constexpr (L >= 2) v = op(v, dpp_move<0xB1>(v));    // quad_perm [1,0,3,2]: xor 1
    if constexpr (L >= 4) v = op(v, dpp_move<0x4E>(v));    // quad_perm [2,3,0,1]: xor 2
    if constexpr (L >= 8) v = op(v, dpp_move<0x141>(v));   // row_half_mirror: 7 - i within 8
    if constexpr (L >= 16) v = op(v, dpp_move<0x140>(v));  // row_mirror: 15 - i within 16
    return v;
}
template <int L>
__device__ __forceinline__ float lane_group_sum(float v) {
    return __builtin_bit_cast(float, lane_group_reduce<L>(__builtin_bit_cast(uint32_t, v),
        [](uint32_t a, uint32_t b) {
            return __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
        }));
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) {
    return __builtin_bit_cast(half2_t, u);
}
__device__ __forceinline__ uint32_t as_u32(half2_t h) {
    return __builtin_bit_cast(uint32_t, h);
}

// Exact dequantization of a biased pair: (1024+q) - (1024+z) is the exact small
// integer q - z, and the single fp16 multiply by s rounds once to nearest even,
// so each half equals fp16_rne(s * (q - z)).
__device__ __forceinline__ uint32_t dequant_pair(uint32_t p, half2_t bz2, half2_t s2) {
    return as_u32((as_half2(p) - bz2) * s2);
}

// (lo(a), lo(b)) and (hi(a), hi(b)) as one 32-bit half2 each, one v_perm_b32
// apiece (selector bytes 0-3 pick bytes of the second operand, 4-7 of the first).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Pairs in (j, j+4) order -> eight halves in natural k order (as four dwords).
__device__ __forceinline__ uint4 pairs_to_natural(const uint32_t d[4]) {
    uint4 n;
    n.x = pack_lo(d[0], d[1]);  // (w0, w1)
    n.y = pack_lo(d[2], d[3]);  // (w2, w3)
    n.z = pack_hi(d[0], d[1]);  // (w4, w5)
    n.w = pack_hi(d[2], d[3]);  // (w6, w7)
    return n;
}

// Eight halves in natural k order -> (j, j+4) pair order, the inverse of the above.
__device__ __forceinline__ uint4 natural_to_pairs(uint4 x) {
    uint4 a;
    a.x = pack_lo(x.x, x.z);  // (x0, x4)
    a.y = pack_hi(x.x, x.z);  // (x1, x5)
    a.z = pack_lo(x.y, x.w);  // (x2, x6)
    a.w = pack_hi(x.y, x.w);  // (x3, x7)
    return a;
}

// Exact dequantization of one qweight word to eight halves in natural k order.
// bz = 1024 + zero as fp16, s = scale, mask = kNibblePairMask.
__device__ __forceinline__ uint4 dequant_word_natural(uint32_t w, uint32_t mask, half_t bz,
                                                      half_t s) {
    uint32_t p[4], d[4];
    unpack_biased(w, mask, p);
    const half2_t bz2 = {bz, bz};
    const half2_t s2 = {s, s};
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = dequant_pair(p[j], bz2, s2);
    return pairs_to_natural(d);
}

// ---------------------------------------------------------------------------
// Kernel-private interleaved words (the layout awq_repack makes): the code of
// k = 8r + j sits at nibble 4 (j % 2) + j / 2, i.e. the even k of the word in
// the low half-word (k 2i at nibble i) and the odd k in the high half-word
// (k 2i + 1 at nibble 4 + i).  Each natural-order pair (k 2e, k 2e + 1) is then
// at the same bit of the two half-words.
constexpr uint32_t kHighNibblePairMask = 0x00F000F0u;
// fp16 0x5400 | (c << 4) is exactly 64 + c: exponent 2^6, ulp 1/16, so a nibble
// at bits 4..7 of a half counts units.
constexpr uint32_t kBias64x2 = 0x54005400u;

// The high-nibble pair mask in a vector register (see nibble_mask_vgpr).
__device__ __forceinline__ uint32_t high_mask_vgpr() {
    uint32_t v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(kHighNibblePairMask));
    return v;
}

// Interleaved word -> the four natural-order pairs
//   p[e] = (b_e + q_2e, b_e + q_2e+1),  b_e = 1024 for even e, 64 for odd e,
// with one shift and four AND-ORs.  lo_mask / hi_mask: kNibblePairMask and
// kHighNibblePairMask, in vector registers.
__device__ __forceinline__ void unpack_interleaved(uint32_t w, uint32_t lo_mask, uint32_t hi_mask,
                                                   uint32_t p[4]) {
    const uint32_t w8 = w >> 8;
    p[0] = (w & lo_mask) | kBias1024x2;
    p[1] = (w & hi_mask) | kBias64x2;
    p[2] = (w8 & lo_mask) | kBias1024x2;
    p[3] = (w8 & hi_mask) | kBias64x2;
}

// Bytes (0, 2, 1, 3) of w: swaps the middle two bytes.
__device__ __forceinline__ uint32_t swap_middle_bytes(uint32_t w) {
    return __builtin_amdgcn_perm(w, w, 0x03010200u);
}
// Swaps nibbles 1 and 2 of each half-word.
__device__ __forceinline__ uint32_t swap_middle_nibbles(uint32_t w) {
    const uint32_t d = ((w >> 4) ^ w) & 0x00F000F0u;
    return w ^ d ^ (d << 4);
}
// Interleaved word -> canonical word (code j at nibble j), and back.  The
// half-words of an interleaved word hold (k0 k2 k4 k6 | k1 k3 k5 k7); after the
// byte swap they hold (k0 k2 k1 k3 | k4 k6 k5 k7), and the nibble swap gives
// (k0 k1 k2 k3 | k4 k5 k6 k7).
__device__ __forceinline__ uint32_t deinterleave_word(uint32_t w) {
    return swap_middle_nibbles(swap_middle_bytes(w));
}
__device__ __forceinline__ uint32_t interleave_word(uint32_t w) {
    return swap_middle_bytes(swap_middle_nibbles(w));
}

// Where the packed words sit.  The kernels take the qweight layout as a
// template parameter IL: 0 canonical, 1 interleaved, 2 blocked (see
// include/awq.h); a nonzero IL means interleaved nibble order.  In the blocked
// layout the columns are cut into blocks of kQBlock, and block b stores packed
// row 0 of its columns, then row 1, and so on: word (r, n) sits at
//   (n / kQBlock) * KR * kQBlock + r * kQBlock + n % kQBlock   (KR = K / 8).
// A run of columns inside one block is contiguous in both layouts, so every
// kernel load (at most 8 words, aligned to its width) stays one load.
constexpr int kQBlock = 128;
constexpr bool blocked_layout(int il) { return il == 2; }
// Words between packed rows r and r + 1 of one column.
__host__ __device__ __forceinline__ int q_pitch(bool blk, int N) { return blk ? kQBlock : N; }
// Offset of word (0, n), in words.
__host__ __device__ __forceinline__ uint32_t q_col(bool blk, int n, int KR) {
    return blk ? (uint32_t)(n / kQBlock) * (uint32_t)KR * (uint32_t)kQBlock +
                     (uint32_t)(n % kQBlock)
               : (uint32_t)n;
}

// 1024 + z as fp16, from the 4-bit zero point z.
__device__ __forceinline__ half_t biased_zero(uint32_t z) {
    return __builtin_bit_cast(half_t, (uint16_t)(0x6400u | (z & 0xFu)));
}

__device__ __forceinline__ half_t as_half(uint16_t u) {
    return __builtin_bit_cast(half_t, u);
}
__device__ __forceinline__ uint16_t as_u16(half_t h) {
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ half8_t as_half8(uint4 u) {
    return __builtin_bit_cast(half8_t, u);
}

}  // namespace awq
