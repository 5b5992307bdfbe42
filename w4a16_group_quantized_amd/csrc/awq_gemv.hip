// Fused W4A16 dequantize-and-multiply for small batches (1 <= M <= 16), the
// decode-time matrix-vector product of AWQ's WQLinear_GEMV module (pyshine.com
// AutoAWQ tour, overview bullets; unfragile.ai AutoAWQ page, the WQLinear
// paragraph).  This file picks the kernel family for a shape; the kernels and
// their design are in awq_gemv_kernels.h, one family per awq_gemv_*.hip file.
#include "awq_gemv_kernels.h"

namespace awq {

hipError_t launch_gemv(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                       const int32_t *qzeros, uint16_t *y, int M, int K, int N, int G, int il,
                       hipStream_t s) {
    using namespace gemv;
    // Per-wave staged X, D-deep load pipeline.  The strip width depends on the
    // layer.  On narrow layers, where 64-column strips would leave half the
    // CUs or more idle, 32-column strips (4096 x 4096 at 1 row: 5.9 -> 4.7 us;
    // 14336 x 4096 at 1 row: 16.1 -> 11.0 us).
    const int cus = device_cus();
    const long long n64 = (N + 63) / 64, n128 = (N + 127) / 128;
    const bool narrow = n64 * 2 <= cus;
    // A family's launcher for the layer's word layout (AWQ_LAYOUT_*: 0, 1, 2).
    auto run = [&](Launcher *canon, Launcher *inter, Launcher *blk) {
        return (il == 2 ? blk : il ? inter : canon)(x, qweight, scales, qzeros, y, M, K, N, G, s);
    };
    // Wide layers (128 columns per workgroup still keep three quarters of the
    // CUs busy) with N a multiple of 16, from three rows up: paired strips, 64
    // columns of each half of the layer per workgroup, X staged segment by
    // segment (prog_w8).  Against one 128-column strip on the same words,
    // outputs bit-identical: 4096 x 28672 at 8 rows 14.42 -> 12.62 us (it
    // took 64-column strips there), at 16 rows 15.86 -> 13.94 us; 8192 x
    // 28672 at 8 rows 24.19 -> 22.40 us, at 16 rows 28.24 -> 23.78 us.  At
    // three and four rows, against X staged up front on 64-column strips
    // (the segment sums then come from the matrix cores): 13.65 -> 12.13 and
    // 13.57 -> 12.76 us; 22.46 -> 21.04 and 22.55 -> 21.75 us.  At one and two
    // rows, and as two 32-column strips with 8-byte loads, they do not pay.
    const bool pair = N % 16 == 0 && n128 * 4 >= 3LL * cus;
    if (M > 2 && pair && stream_fits_prog(M, K, N, G, 8, 8, 1))
        return run(prog_w8, prog_w8_il, prog_w8_blk);
    if (M > 4) {
        // Beyond four rows X is staged segment by segment, one segment in
        // flight per wave, which takes any K.  Every workgroup reads all of X
        // (M K 2 bytes) beside its strip, so 128-column strips, half as many
        // workgroups, pay where they still keep three quarters of the CUs
        // busy and X is large (4096 x 28672 at 16 rows: 17.1 against 18.9
        // us); else 64-column strips (4096 x 14336 at 16 rows: 9.9 against
        // 15.5 us).
        const bool wide = n128 * 4 >= 3LL * cus && (M > 8 || n64 > 2LL * cus);
        if (narrow && stream_fits_prog(M, K, N, G, 2, 8, 1))
            return run(prog_w2, prog_w2_il, prog_w2_blk);
        if (!wide && stream_fits_prog(M, K, N, G, 4, 8, 1))
            return run(prog_w4, prog_w4_il, prog_w4_blk);
        if (stream_fits_prog(M, K, N, G, 8, 8, 1))
            return run(prog_w8, prog_w8_il, prog_w8_blk);
    }
    if (narrow && stream_fits(M, K, N, G, 2, 8, 16, 2))
        return run(stream_m_w2_d2, stream_m_w2_d2_il, stream_m_w2_d2_blk);
    if (stream_fits(M, K, N, G, 4, 8, 16, 2))
        return run(stream_m_w4_d2, stream_m_w4_d2_il, stream_m_w4_d2_blk);
    if (stream_fits(M, K, N, G, 4, 8, 16, 1))
        return run(stream_m_w4_d1, stream_m_w4_d1_il, stream_m_w4_d1_blk);
    // Up to four rows with X beyond LDS: staged segment by segment as well.
    if (narrow && stream_fits_prog(M, K, N, G, 2, 8, 1))
        return run(prog_w2, prog_w2_il, prog_w2_blk);
    if (stream_fits_prog(M, K, N, G, 4, 8, 1))
        return run(prog_w4, prog_w4_il, prog_w4_blk);
    // A segment (SEGR packed rows) must sit inside one group and be whole 32-k steps.
    // Narrow layers on 32-column strips here too (14336 x 4096 at 16 rows:
    // 27.4 -> 22.1 us).
    if (narrow && G % 128 == 0)
        return fold_w2_s16(x, qweight, scales, qzeros, y, M, K, N, G, il, s);
    if (G % 128 == 0) return fold_w4_s16(x, qweight, scales, qzeros, y, M, K, N, G, il, s);
    if (G % 64 == 0) return fold_w4_s8(x, qweight, scales, qzeros, y, M, K, N, G, il, s);
    if (G % 32 == 0) return fold_w4_s4(x, qweight, scales, qzeros, y, M, K, N, G, il, s);
    return exact_w4(x, qweight, scales, qzeros, y, M, K, N, G, il, s);
}

}  // namespace awq
