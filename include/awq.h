/*
 * awq.h -- C ABI of the MI355X (gfx950) W4A16 group-quantized linear layer.
 *
 * The layer is the inference hot path of AWQ (activation-aware 4-bit weight
 * quantization): Y[M][N] = X[M][K] * W[K][N], where W is kept as 4-bit codes
 * and dequantized inside the multiplication.  Sources on the AWQ pages:
 *   - the quantized linear modules perform INT4 weight dequantization and the
 *     matrix multiplication in one fused kernel, never materializing the fp16
 *     weight, with a matrix-vector variant for single-token decoding and a
 *     GEMM variant for batches (unfragile.ai AutoAWQ page, the WQLinear
 *     paragraph; pyshine.com AutoAWQ tour, the overview bullets on
 *     WQLinear_GEMM / WQLinear_GEMV);
 *   - eight 4-bit weights share one INT32 word, with fp16 scales and zero
 *     points shared by groups of 128 weights (mbrenndoerfer.com,
 *     "AWQ > Implementation", "Understanding the Quantization Structure");
 *   - symmetric dequantization weight = scale * (code - 8) (fak explainer,
 *     "Format Specification > Dequantization Formula"), and one matrix-vector
 *     plus one batched call over a quantized tensor (fak explainer,
 *     "Integration with Forward Pass").
 *
 * Data layout (row-major, dense; fp16 = IEEE binary16 bit patterns):
 *   qweight  int32 [K/8][N]    code of (k, n) in bits 4*(k%8)..4*(k%8)+3 of
 *                              word [k/8][n]: eight consecutive k of one column
 *   scales   fp16  [K/G][N]    scale of group g = k / G for column n
 *   qzeros   int32 [K/G][N/8]  zero of (g, n) in bits 4*(n%8).. of word
 *                              [g][n/8]; NULL selects the symmetric zero 8
 *   x        fp16  [M][K]      activations;   y  fp16 [M][N]   outputs
 * Dequantized weight: w(k, n) = fp16_rne(scale(g, n) * (code(k, n) - zero(g, n))).
 * Layer output: y = fp16_rne(sum_k x(m, k) * w(k, n)), accumulated in fp32.
 *
 * Shape rules (AWQ_ERROR_SHAPE otherwise): K, N, G > 0; K % 8 == 0;
 * N % 8 == 0; G % 8 == 0; K % G == 0; every array below 2^31 elements.
 * Every call that takes an awq_layer takes it in any qweight layout (see
 * AWQ_LAYOUT_*) with the same results, bit for bit where the call is exact.
 * M == 0 is an empty batch: success, nothing launched.  M < 0 is invalid.
 *
 * Pointers: every tensor pointer is a DEVICE pointer, 16-byte aligned
 * (AWQ_ERROR_ALIGNMENT otherwise), owned by the caller, and only read or
 * written while the launched kernels run; the library keeps none of them,
 * allocates no memory and holds no state.  Outputs must not overlap inputs.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  Every call validates its arguments on the host, returns an error
 * code with nothing launched if they are wrong, and otherwise enqueues its
 * kernels and returns without waiting.  A fault inside a kernel surfaces at the
 * caller's next synchronization, as HIP reports it.  Calls are thread safe.
 *
 * Debugging: with AWQ_SYNC set in the environment to anything but "" or "0"
 * (read once, at the first call), every call that launched work waits for its
 * stream before returning and reports a failure of its own kernels as
 * AWQ_ERROR_HIP.  A stream being captured into a graph is not waited for.
 */
#ifndef AWQ_MI355X_H
#define AWQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum awq_status {
    AWQ_SUCCESS = 0,
    AWQ_ERROR_INVALID_VALUE = 1, /* null pointer, negative M, non-positive K/N/G */
    AWQ_ERROR_SHAPE = 2,         /* a shape rule above is broken               */
    AWQ_ERROR_ALIGNMENT = 3,     /* a tensor pointer is not 16-byte aligned    */
    AWQ_ERROR_UNSUPPORTED = 4,   /* valid layer, but outside this entry point (gemv: M > 16) */
    AWQ_ERROR_WORKSPACE = 5,     /* workspace NULL, unaligned or too small      */
    AWQ_ERROR_HIP = 6            /* the HIP runtime refused the launch          */
} awq_status;

/*
 * Layouts of qweight.  AWQ_LAYOUT_CANONICAL is the layout above.
 * AWQ_LAYOUT_INTERLEAVED is a kernel-private repacking of the same words
 * (faster to unpack in the batched kernel; the pages name such formats,
 * GEMVFast and Marlin, in pyshine.com's AutoAWQ tour, "The Quantization Flow
 * Up Close", without giving one): the code of k = 8r + j sits in nibble
 * 4 (j % 2) + j / 2 of word [r][n] -- the even k in the low half-word, the odd
 * k in the high half-word.  AWQ_LAYOUT_BLOCKED holds the interleaved words,
 * moved so that each block of 128 columns is one contiguous run: word [r][n]
 * sits at index (n / 128) * (K / 8) * 128 + r * 128 + n % 128 of the int32
 * array, which keeps its size K/8 * N.  A kernel that streams one strip of
 * columns over all of K then reads one run per block instead of a short piece
 * of every row.  It needs N % 128 == 0 (AWQ_ERROR_SHAPE otherwise).
 * awq_repack converts between any two layouts.
 */
#define AWQ_LAYOUT_CANONICAL 0
#define AWQ_LAYOUT_INTERLEAVED 1
#define AWQ_LAYOUT_BLOCKED 2

/* Non-owning view of one quantized linear layer (logical weight W[K][N]).
 * A zero-initialized layout field is the canonical layout. */
typedef struct awq_layer {
    const int32_t *qweight;      /* [K/8][N] in `layout`                       */
    const uint16_t *scales;      /* [K/G][N] fp16                              */
    const int32_t *qzeros;       /* [K/G][N/8], or NULL for symmetric (zero 8) */
    int32_t K;
    int32_t N;
    int32_t group_size;          /* G; G == K gives one scale per column        */
    int32_t layout;              /* AWQ_LAYOUT_*; any other value is AWQ_ERROR_INVALID_VALUE */
} awq_layer;

/* Human-readable name of a status code (static storage, never NULL). */
const char *awq_status_string(awq_status status);

/*
 * awq_pack: codes uint8 [K][N] (one 4-bit code per byte; bits above the low
 * nibble are ignored) -> qweight int32 [K/8][N].  The packing of eight 4-bit
 * weights into one INT32 word is the mbrenndoerfer.com "Understanding the
 * Quantization Structure" layout; done once per layer, when it is loaded.
 */
awq_status awq_pack(const uint8_t *codes, int32_t *qweight, int32_t K, int32_t N,
                    void *stream);

/*
 * awq_pack_zeros: zeros uint8 [groups][N] -> qzeros int32 [groups][N/8],
 * eight consecutive columns per word, zero of column 8c + j in bits 4j..4j+3
 * of word c (bits above the low nibble of each byte are ignored).  groups =
 * K / G.  The layer stores one zero point per group beside its scale, and
 * asymmetric quantization (zero_point=True) uses them (mbrenndoerfer.com,
 * "AWQ > Implementation", "Understanding the Quantization Structure": the
 * qzeros tensor; pyshine.com AutoAWQ tour, "From Install to Your First
 * Model": zero_point).  Done once per layer, when it is loaded.
 */
awq_status awq_pack_zeros(const uint8_t *zeros, int32_t *qzeros, int32_t groups,
                          int32_t N, void *stream);

/*
 * awq_repack: packed words qweight [K/8][N] from layout `from` to layout `to`
 * (AWQ_LAYOUT_*; from == to copies).  A fixed permutation of the nibbles of
 * each word, and of the words' places for the blocked layout, done once per
 * layer when it is loaded: the kernel-private layouts of the pages' faster
 * kernels are such repackings of the packed weight (pyshine.com AutoAWQ tour,
 * "The Quantization Flow Up Close": GEMVFast, Marlin, unpack_reorder_pack).
 * src and dst: device int32 arrays of K/8 * N words, 16-byte aligned, not
 * overlapping, except that dst may equal src (in place) when neither or both
 * layouts are blocked; in place across the blocked layout is
 * AWQ_ERROR_INVALID_VALUE.  K % 8 == 0, N % 8 == 0 (N % 128 == 0 if either
 * layout is blocked), K * N below 2^31 (AWQ_ERROR_SHAPE otherwise); an unknown
 * layout is AWQ_ERROR_INVALID_VALUE.
 */
awq_status awq_repack(const int32_t *src, int32_t *dst, int32_t K, int32_t N, int32_t from,
                      int32_t to, void *stream);

/*
 * awq_dequant: materializes W[K][N] fp16 from the layer, bit-exactly
 * w = fp16_rne(scale * (code - zero)): the weight of a code is its scale times
 * its distance from the zero point, 8 in the symmetric form (fak explainer,
 * "Format Specification > Dequantization Formula"; with the stored per-group
 * zero points of mbrenndoerfer.com, "AWQ > Implementation", "Understanding
 * the Quantization Structure").  Not on the decode path (the fused kernels
 * never write W); it exposes the exact dequantization the fused kernels
 * perform.  w_out: device fp16 [K][N], 16-byte aligned (AWQ_ERROR_ALIGNMENT);
 * NULL is AWQ_ERROR_INVALID_VALUE.
 */
awq_status awq_dequant(const awq_layer *layer, uint16_t *w_out, void *stream);

/*
 * awq_gemv: fused dequantize-and-multiply for small batches, 1 <= M <= 16 (the
 * pages' matrix-vector module for single-token decoding: pyshine.com AutoAWQ
 * tour, the overview bullet on WQLinear_GEMM / WQLinear_GEMV; fak explainer, "Integration with Forward
 * Pass": one matrix-vector call over a quantized tensor).  Streams the packed
 * weight once.  M > 16 returns AWQ_ERROR_UNSUPPORTED; use awq_gemm.
 *   x: device fp16 [M][K];  y: device fp16 [M][N], 16-byte aligned.
 *   workspace: device scratch of at least awq_gemv_workspace_bytes(M, K, N)
 *     bytes, owned by the caller.  The query returns 0 for every shape (the
 *     K-split partial sums are reduced inside each workgroup, through LDS), so
 *     workspace may be NULL with workspace_bytes 0; a non-NULL workspace must
 *     be 16-byte aligned (AWQ_ERROR_WORKSPACE otherwise).  It is never read or
 *     written.
 */
size_t awq_gemv_workspace_bytes(int32_t M, int32_t K, int32_t N);

awq_status awq_gemv(const uint16_t *x, const awq_layer *layer, uint16_t *y, int32_t M,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * awq_gemm: fused dequantize-and-multiply for any M >= 0 (the pages' GEMM
 * module for batched inference): weights are dequantized tile by tile into
 * on-chip memory and multiplied with fp16 matrix-core instructions, fp32
 * accumulation.  Each weight is dequantized exactly as awq_dequant does,
 * except on one-group layers (group_size == K): there the matrix cores take
 * q - z (exact) and each column's scale multiplies its fp32 sum once, as
 * awq_gemv does per group (no fp16 rounding of each s (q - z); the difference
 * is far inside the layer's output tolerance).
 */
awq_status awq_gemm(const uint16_t *x, const awq_layer *layer, uint16_t *y, int32_t M,
                    void *stream);

/*
 * awq_quantize: produces a layer from fp16 weights, the step before the fused
 * kernels (the pages' pseudo-quantization pass rounds each group of weights to
 * integer levels against a scale and zero point: pyshine.com AutoAWQ tour,
 * "The Quantization Flow Up Close"; zero_point / q_group_size / w_bit in
 * "From Install to Your First Model").  Per group of G rows and column n,
 * textbook min-max:
 *   asymmetric (symmetric == 0): r = hi - lo (|hi| for a constant group),
 *       s = fp16(r / 15), z = clamp(rint(-lo / s), 0, 15)
 *   symmetric (symmetric != 0): s = fp16(max|w| / 7), zero point 8
 *   both: s = 1 if it rounds to 0; code = clamp(rint(w / s) + z, 0, 15)
 * lo, hi: the group's minimum and maximum.  The scale is the exact real
 * r / 15 (or r / 7) rounded once to fp16 (round to nearest even); z and the
 * codes are decided in fp32 (correctly rounded division, round to nearest
 * even).  Weights must be finite.
 *   w: device fp16 [K][N].  Outputs as in awq_layer: qweight int32 [K/8][N],
 *   scales fp16 [K/G][N], qzeros int32 [K/G][N/8] (not written, and may be
 *   NULL, when symmetric).  Shape and alignment rules are the layer's.
 */
awq_status awq_quantize(const uint16_t *w, int32_t K, int32_t N, int32_t group_size,
                        int32_t symmetric, int32_t *qweight, uint16_t *scales, int32_t *qzeros,
                        void *stream);

/*
 * awq_gemv_gate_up: the fused MLP front of a Llama-style block in one pass.
 * The inference stack concatenates the gate and up projections into one
 * quantized MLP module (pyshine.com AutoAWQ tour, the introduction and "The
 * Quantization Flow Up Close": QuantFusedMLP); the Llama-family MLP then
 * multiplies SiLU(gate) by up (unfragile.ai AutoAWQ page, the Llama/Mistral
 * paragraph).
 *
 * The layer holds the concatenation: its N = 2I columns are [gate | up]
 * (columns n < I the gate projection, I + n the up projection of the same
 * output n), packed, scaled and zeroed like any layer.  The output is
 *     h[m][n] = fp16_rne(SiLU(y(m, n)) * y(m, I + n)),   n < I,
 * with y the layer's fp32 sums (never rounded to fp16 on the way) and
 * SiLU(t) = t / (1 + e^-t) in fp32.  Y is never written.
 *   x: device fp16 [M][K];  h: device fp16 [M][I], 16-byte aligned.
 * Rules beyond the layer's: 1 <= M <= 16 (M == 0 is a no-op); N % 16 == 0
 * (I a multiple of 8).  Shapes the fused kernel does not cover return
 * AWQ_ERROR_UNSUPPORTED with nothing launched: G must be a multiple of 128.
 * Any K: an X too large for LDS is staged segment by segment.
 */
awq_status awq_gemv_gate_up(const uint16_t *x, const awq_layer *layer, uint16_t *h, int32_t M,
                            void *stream);

/*
 * awq_gemm_gate_up: the same fused gate/up output as awq_gemv_gate_up, for any
 * batch (M >= 0), on the batched GEMM path: the layer's N = 2I columns are
 * [gate | up] and h[m][n] = fp16_rne(SiLU(y(m, n)) * y(m, I + n)), n < I, from
 * the fp32 sums, with each weight dequantized exactly as awq_dequant does.
 *   x: device fp16 [M][K];  h: device fp16 [M][I], 16-byte aligned.
 * Rules beyond the layer's: N % 16 == 0.  Shapes outside the fused GEMM
 * kernel return AWQ_ERROR_UNSUPPORTED before any launch: G must be a multiple
 * of 64 and K a multiple of 256.
 */
awq_status awq_gemm_gate_up(const uint16_t *x, const awq_layer *layer, uint16_t *h, int32_t M,
                            void *stream);

/*
 * awq_gemm_splitk: the same output as awq_gemm, for batches too small to fill
 * the GPU with output tiles (roughly M up to a few hundred rows at K = 4096):
 * K is cut into `splits` slices, each summed by its own workgroups with the
 * weights dequantized as awq_gemm does, into fp32 partial outputs
 * in `workspace`; the slices are then added in order and rounded once to fp16
 * (deterministic).  splits == 1 is awq_gemm (workspace ignored).
 *   x: device fp16 [M][K];  y: device fp16 [M][N], 16-byte aligned.
 *   splits: 1..16 (AWQ_ERROR_INVALID_VALUE otherwise); K % splits == 0 and each
 *     slice a whole number of groups (or G == K) and of 256 k (or 128 k with G
 *     a multiple of 32), else AWQ_ERROR_UNSUPPORTED before any launch.
 *   workspace: device memory of at least awq_gemm_splitk_workspace_bytes(M, N,
 *     splits) bytes (splits * M * N fp32), 16-byte aligned, owned by the
 *     caller (AWQ_ERROR_WORKSPACE otherwise); its contents on return are
 *     unspecified.
 */
size_t awq_gemm_splitk_workspace_bytes(int32_t M, int32_t N, int32_t splits);

awq_status awq_gemm_splitk(const uint16_t *x, const awq_layer *layer, uint16_t *y, int32_t M,
                           int32_t splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * awq_gemm_splitk_static: awq_gemm_splitk without a caller workspace and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The fp32 partial outputs go into a static scratch array of
 * AWQ_GEMM_SPLITK_STATIC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on, from the first call there until the process ends; the call itself
 * allocates nothing.  Same arguments, rules and output as awq_gemm_splitk
 * (bit-identical: the same kernels), except that splits * M * N * 4 bytes
 * above the scratch size return AWQ_ERROR_WORKSPACE before any launch.
 * All calls on one GPU share its scratch: calls that overlap in time on one
 * GPU (two streams, two host threads) race and give undefined outputs.
 */
#define AWQ_GEMM_SPLITK_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

awq_status awq_gemm_splitk_static(const uint16_t *x, const awq_layer *layer, uint16_t *y,
                                  int32_t M, int32_t splits, void *stream);

/*
 * The scale search of AWQ's calibration (pyshine.com AutoAWQ tour, "The
 * Quantization Flow Up Close": per-channel means of normalized weights and of
 * activations, the FP16 module run once as the reference, the candidate
 * scaling of least output error; scale_ln_fcs: dividing the preceding op's
 * output by c and multiplying the weights by c leaves the layer unchanged
 * before rounding).  The pages give no formula for the statistics, the
 * candidates or the grid; the readings taken are:
 *   xbar[k] = mean over calibration rows of |x(m, k)|;
 *   wbar[k] = mean over output columns n of |w(k, n)| / a(g, n), with a(g, n)
 *             the largest |w| of k's quantization group in column n (an
 *             all-zero group adds 0);
 *   c[k]    = max(xbar[k], 1e-4)^alpha / max(wbar[k], 1e-4)^(1 - alpha);
 *   loss(alpha) = mean over (m, n) of (y - y')^2, with y = x W in fp32 and
 *             y' the awq_gemm output for fp16(x / c) and the layer that
 *             awq_quantize makes of fp16(c W); the first alpha of least loss
 *             is kept.
 *
 * Inputs: x device fp16 [M][K] calibration activations (M >= 1), w device fp16
 * [K][N] the layer's unquantized weight, both 16-byte aligned; the layer's
 * shape rules apply, and M*K, K*N and M*N must be below 2^31.
 * Workspace: device memory of at least the *_workspace_bytes query for the
 * same sizes, 16-byte aligned, owned by the caller; its contents on return are
 * unspecified.  AWQ_ERROR_WORKSPACE if it is NULL, unaligned or too small.
 * Both calls enqueue on `stream` and return without waiting.  Results are
 * deterministic: every reduction runs in a fixed order.
 */
size_t awq_channel_stats_workspace_bytes(int32_t M, int32_t K, int32_t N, int32_t group_size);

/* xbar, wbar: device fp32 [K] outputs (4-byte aligned). */
awq_status awq_channel_stats(const uint16_t *x, int32_t M, const uint16_t *w, int32_t K, int32_t N,
                             int32_t group_size, float *xbar, float *wbar, void *workspace,
                             size_t workspace_bytes, void *stream);

size_t awq_scale_search_workspace_bytes(int32_t M, int32_t K, int32_t N, int32_t group_size);

/*
 * alphas: HOST array of n_alpha grid values in [0, 1], 1 <= n_alpha <= 64
 * (AWQ_ERROR_INVALID_VALUE otherwise, NaN included); read before the call
 * returns.  losses: device fp64 [n_alpha]; best: device int32, the index of the
 * first least loss; best_scales: device fp32 [K], the scales c of that alpha,
 * or NULL.  symmetric != 0 quantizes the migrated weight with the symmetric
 * zero 8.
 */
awq_status awq_scale_search(const uint16_t *x, int32_t M, const uint16_t *w, int32_t K, int32_t N,
                            int32_t group_size, int32_t symmetric, const float *alphas,
                            int32_t n_alpha, double *losses, int32_t *best, float *best_scales,
                            void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_H */
