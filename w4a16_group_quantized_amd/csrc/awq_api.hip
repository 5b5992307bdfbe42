// C ABI of libawq (declared in include/awq.h): argument validation on the
// host, then one launch on the caller's stream.  Validation runs before any
// HIP call, so a rejected call touches neither the device nor the stream.
#include "../../include/awq.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdlib.h>

#include "awq_internal.h"

namespace {

constexpr long long kMaxElems = (1LL << 31) - 1;
constexpr int kMaxSplits = 16;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

awq_status check_layer(const awq_layer *w) {
    if (w == nullptr || w->qweight == nullptr || w->scales == nullptr)
        return AWQ_ERROR_INVALID_VALUE;
    const long long K = w->K, N = w->N, G = w->group_size;
    if (K <= 0 || N <= 0 || G <= 0) return AWQ_ERROR_INVALID_VALUE;
    if (w->layout != AWQ_LAYOUT_CANONICAL && w->layout != AWQ_LAYOUT_INTERLEAVED &&
        w->layout != AWQ_LAYOUT_BLOCKED)
        return AWQ_ERROR_INVALID_VALUE;
    if (K % 8 || N % 8 || G % 8 || K % G) return AWQ_ERROR_SHAPE;
    if (w->layout == AWQ_LAYOUT_BLOCKED && N % 128) return AWQ_ERROR_SHAPE;
    if (K * N > kMaxElems) return AWQ_ERROR_SHAPE;  // the dequantized weight's element count
    if (!aligned16(w->qweight) || !aligned16(w->scales) ||
        (w->qzeros != nullptr && !aligned16(w->qzeros)))
        return AWQ_ERROR_ALIGNMENT;
    return AWQ_SUCCESS;
}

awq_status check_io(const uint16_t *x, const uint16_t *y, const awq_layer *w, int32_t M) {
    if (M < 0) return AWQ_ERROR_INVALID_VALUE;
    if (M == 0) return AWQ_SUCCESS;
    if (x == nullptr || y == nullptr) return AWQ_ERROR_INVALID_VALUE;
    if ((long long)M * w->K > kMaxElems || (long long)M * w->N > kMaxElems) return AWQ_ERROR_SHAPE;
    if (!aligned16(x) || !aligned16(y)) return AWQ_ERROR_ALIGNMENT;
    return AWQ_SUCCESS;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// AWQ_SYNC set to anything but "" or "0" in the environment (read once, at the
// first call): every call that launched work waits for its stream and reports
// a fault of its own kernels as AWQ_ERROR_HIP, instead of leaving it to the
// caller's next synchronization.  A stream that is being captured into a graph
// is not waited for (a capture cannot synchronize).  For debugging only: the
// wait serializes the caller with the GPU.
bool sync_mode() {
    static const bool on = [] {
        const char *v = getenv("AWQ_SYNC");
        return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
    }();
    return on;
}

// The status of a call whose launches returned e on `stream`.
awq_status done(void *stream, hipError_t e) {
    if (e != hipSuccess) return AWQ_ERROR_HIP;
    if (!sync_mode()) return AWQ_SUCCESS;
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(as_stream(stream), &capture) != hipSuccess) return AWQ_ERROR_HIP;
    if (capture != hipStreamCaptureStatusNone) return AWQ_SUCCESS;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return AWQ_ERROR_HIP;
    return hipGetLastError() == hipSuccess ? AWQ_SUCCESS : AWQ_ERROR_HIP;
}

// The launchers take the layout as AWQ_LAYOUT_* (checked by check_layer).
int layout_of(const awq_layer *w) { return w->layout; }

// Calibration X [M][K] and fp16 weight W [K][N] of the scale search.
awq_status check_calibration(const uint16_t *x, int32_t M, const uint16_t *w, int32_t K, int32_t N,
                             int32_t G) {
    if (x == nullptr || w == nullptr || M <= 0 || K <= 0 || N <= 0 || G <= 0)
        return AWQ_ERROR_INVALID_VALUE;
    if (K % 8 || N % 8 || G % 8 || K % G) return AWQ_ERROR_SHAPE;
    if ((long long)M * K > kMaxElems || (long long)K * N > kMaxElems || (long long)M * N > kMaxElems)
        return AWQ_ERROR_SHAPE;
    if (!aligned16(x) || !aligned16(w)) return AWQ_ERROR_ALIGNMENT;
    return AWQ_SUCCESS;
}

}  // namespace

extern "C" {

const char *awq_status_string(awq_status status) {
    switch (status) {
    case AWQ_SUCCESS: return "AWQ_SUCCESS";
    case AWQ_ERROR_INVALID_VALUE: return "AWQ_ERROR_INVALID_VALUE: null pointer or non-positive size";
    case AWQ_ERROR_SHAPE: return "AWQ_ERROR_SHAPE: K%8, N%8, G%8, K%G must be 0 (and N%128 in the blocked layout) and arrays below 2^31 elements";
    case AWQ_ERROR_ALIGNMENT: return "AWQ_ERROR_ALIGNMENT: tensor pointers must be 16-byte aligned";
    case AWQ_ERROR_UNSUPPORTED: return "AWQ_ERROR_UNSUPPORTED: outside this entry point (awq_gemv takes M <= 16; awq_gemv_gate_up also needs G % 128 == 0; awq_gemm_gate_up needs G % 64 == 0 and K % 256 == 0; awq_gemm_splitk needs slices of whole groups (or one group) and whole 128- or 256-k ring turns)";
    case AWQ_ERROR_WORKSPACE: return "AWQ_ERROR_WORKSPACE: null, unaligned or smaller than the *_workspace_bytes query";
    case AWQ_ERROR_HIP: return "AWQ_ERROR_HIP: the HIP runtime refused the launch";
    }
    return "AWQ_ERROR_UNKNOWN";
}

awq_status awq_pack(const uint8_t *codes, int32_t *qweight, int32_t K, int32_t N, void *stream) {
    if (codes == nullptr || qweight == nullptr || K <= 0 || N <= 0) return AWQ_ERROR_INVALID_VALUE;
    if (K % 8 || N % 8 || (long long)K * N > kMaxElems) return AWQ_ERROR_SHAPE;
    if (!aligned16(codes) || !aligned16(qweight)) return AWQ_ERROR_ALIGNMENT;
    return done(stream, awq::launch_pack(codes, qweight, K, N, as_stream(stream)));
}

awq_status awq_pack_zeros(const uint8_t *zeros, int32_t *qzeros, int32_t groups, int32_t N,
                          void *stream) {
    if (zeros == nullptr || qzeros == nullptr || groups <= 0 || N <= 0)
        return AWQ_ERROR_INVALID_VALUE;
    if (N % 8 || (long long)groups * N > kMaxElems) return AWQ_ERROR_SHAPE;
    if (!aligned16(zeros) || !aligned16(qzeros)) return AWQ_ERROR_ALIGNMENT;
    return done(stream, awq::launch_pack_zeros(zeros, qzeros, groups, N, as_stream(stream)));
}

awq_status awq_repack(const int32_t *src, int32_t *dst, int32_t K, int32_t N, int32_t from,
                      int32_t to, void *stream) {
    if (src == nullptr || dst == nullptr || K <= 0 || N <= 0) return AWQ_ERROR_INVALID_VALUE;
    const auto known = [](int32_t l) {
        return l == AWQ_LAYOUT_CANONICAL || l == AWQ_LAYOUT_INTERLEAVED || l == AWQ_LAYOUT_BLOCKED;
    };
    if (!known(from) || !known(to)) return AWQ_ERROR_INVALID_VALUE;
    // In place only where no word moves: the blocked layout moves words.
    if (src == dst && (from == AWQ_LAYOUT_BLOCKED) != (to == AWQ_LAYOUT_BLOCKED))
        return AWQ_ERROR_INVALID_VALUE;
    if (K % 8 || N % 8 || (long long)K * N > kMaxElems) return AWQ_ERROR_SHAPE;
    if ((from == AWQ_LAYOUT_BLOCKED || to == AWQ_LAYOUT_BLOCKED) && N % 128) return AWQ_ERROR_SHAPE;
    if (!aligned16(src) || !aligned16(dst)) return AWQ_ERROR_ALIGNMENT;
    const long long words = (long long)(K / 8) * N;
    if (from == to) {
        if (src == dst) return AWQ_SUCCESS;
        return done(stream, hipMemcpyAsync(dst, src, (size_t)words * 4, hipMemcpyDeviceToDevice,
                                       as_stream(stream)));
    }
    return done(stream, awq::launch_repack(src, dst, K, N, from, to, as_stream(stream)));
}

awq_status awq_dequant(const awq_layer *layer, uint16_t *w_out, void *stream) {
    awq_status st = check_layer(layer);
    if (st != AWQ_SUCCESS) return st;
    if (w_out == nullptr) return AWQ_ERROR_INVALID_VALUE;
    if (!aligned16(w_out)) return AWQ_ERROR_ALIGNMENT;
    return done(stream, awq::launch_dequant(layer->qweight, layer->scales, layer->qzeros, w_out,
                                        layer->K, layer->N, layer->group_size, layout_of(layer), as_stream(stream)));
}

size_t awq_gemv_workspace_bytes(int32_t M, int32_t K, int32_t N) {
    (void)M;
    (void)K;
    (void)N;
    return 0;   // the K split is reduced inside each workgroup (LDS)
}

awq_status awq_gemv(const uint16_t *x, const awq_layer *layer, uint16_t *y, int32_t M,
                    void *workspace, size_t workspace_bytes, void *stream) {
    awq_status st = check_layer(layer);
    if (st != AWQ_SUCCESS) return st;
    st = check_io(x, y, layer, M);
    if (st != AWQ_SUCCESS || M == 0) return st;
    if (M > 16) return AWQ_ERROR_UNSUPPORTED;
    if (workspace != nullptr && !aligned16(workspace)) return AWQ_ERROR_WORKSPACE;
    if (workspace_bytes < awq_gemv_workspace_bytes(M, layer->K, layer->N)) return AWQ_ERROR_WORKSPACE;
    return done(stream, awq::launch_gemv(x, layer->qweight, layer->scales, layer->qzeros, y, M,
                                     layer->K, layer->N, layer->group_size, layout_of(layer), as_stream(stream)));
}

awq_status awq_gemm(const uint16_t *x, const awq_layer *layer, uint16_t *y, int32_t M,
                    void *stream) {
    awq_status st = check_layer(layer);
    if (st != AWQ_SUCCESS) return st;
    st = check_io(x, y, layer, M);
    if (st != AWQ_SUCCESS || M == 0) return st;
    return done(stream, awq::launch_gemm(x, layer->qweight, layer->scales, layer->qzeros, y, M,
                                     layer->K, layer->N, layer->group_size, layout_of(layer), as_stream(stream)));
}

awq_status awq_quantize(const uint16_t *w, int32_t K, int32_t N, int32_t group_size,
                        int32_t symmetric, int32_t *qweight, uint16_t *scales, int32_t *qzeros,
                        void *stream) {
    if (w == nullptr || qweight == nullptr || scales == nullptr || (!symmetric && qzeros == nullptr))
        return AWQ_ERROR_INVALID_VALUE;
    if (K <= 0 || N <= 0 || group_size <= 0) return AWQ_ERROR_INVALID_VALUE;
    if (K % 8 || N % 8 || group_size % 8 || K % group_size || (long long)K * N > kMaxElems)
        return AWQ_ERROR_SHAPE;
    if (!aligned16(w) || !aligned16(qweight) || !aligned16(scales) ||
        (!symmetric && !aligned16(qzeros)))
        return AWQ_ERROR_ALIGNMENT;
    return done(stream, awq::launch_quantize(w, qweight, scales, qzeros, K, N, group_size,
                                         symmetric != 0, as_stream(stream)));
}

awq_status awq_gemv_gate_up(const uint16_t *x, const awq_layer *layer, uint16_t *h, int32_t M,
                            void *stream) {
    awq_status st = check_layer(layer);
    if (st != AWQ_SUCCESS) return st;
    if (layer->N % 16) return AWQ_ERROR_SHAPE;
    st = check_io(x, h, layer, M);
    if (st != AWQ_SUCCESS || M == 0) return st;
    if (!awq::gemv_gate_up_supported(M, layer->K, layer->N, layer->group_size))
        return AWQ_ERROR_UNSUPPORTED;
    return done(stream, awq::launch_gemv_gate_up(x, layer->qweight, layer->scales, layer->qzeros, h, M,
                                             layer->K, layer->N, layer->group_size,
                                             layout_of(layer), as_stream(stream)));
}

awq_status awq_gemm_gate_up(const uint16_t *x, const awq_layer *layer, uint16_t *h, int32_t M,
                            void *stream) {
    awq_status st = check_layer(layer);
    if (st != AWQ_SUCCESS) return st;
    if (layer->N % 16) return AWQ_ERROR_SHAPE;
    st = check_io(x, h, layer, M);
    if (st != AWQ_SUCCESS || M == 0) return st;
    if (!awq::gemm_gate_up_supported(layer->K, layer->N, layer->group_size))
        return AWQ_ERROR_UNSUPPORTED;
    return done(stream, awq::launch_gemm_gate_up(x, layer->qweight, layer->scales, layer->qzeros, h, M,
                                             layer->K, layer->N, layer->group_size,
                                             layout_of(layer), as_stream(stream)));
}

size_t awq_gemm_splitk_workspace_bytes(int32_t M, int32_t N, int32_t splits) {
    if (M <= 0 || N <= 0 || splits < 1 || splits > kMaxSplits) return 0;
    return awq::gemm_splitk_workspace(M, N, splits);
}

awq_status awq_gemm_splitk(const uint16_t *x, const awq_layer *layer, uint16_t *y, int32_t M,
                           int32_t splits, void *workspace, size_t workspace_bytes, void *stream) {
    awq_status st = check_layer(layer);
    if (st != AWQ_SUCCESS) return st;
    if (splits < 1 || splits > kMaxSplits) return AWQ_ERROR_INVALID_VALUE;
    st = check_io(x, y, layer, M);
    if (st != AWQ_SUCCESS || M == 0) return st;
    if (splits == 1)
        return done(stream, awq::launch_gemm(x, layer->qweight, layer->scales, layer->qzeros, y, M,
                                         layer->K, layer->N, layer->group_size, layout_of(layer), as_stream(stream)));
    if (!awq::gemm_splitk_supported(layer->K, layer->group_size, splits)) return AWQ_ERROR_UNSUPPORTED;
    if ((long long)splits * M * layer->N > kMaxElems) return AWQ_ERROR_SHAPE;
    if (workspace == nullptr || !aligned16(workspace) ||
        workspace_bytes < awq::gemm_splitk_workspace(M, layer->N, splits))
        return AWQ_ERROR_WORKSPACE;
    return done(stream, awq::launch_gemm_splitk(x, layer->qweight, layer->scales, layer->qzeros, y, M,
                                            layer->K, layer->N, layer->group_size, splits, workspace,
                                            layout_of(layer), as_stream(stream)));
}

awq_status awq_gemm_splitk_static(const uint16_t *x, const awq_layer *layer, uint16_t *y,
                                  int32_t M, int32_t splits, void *stream) {
    static_assert(awq::kStaticScratchBytes == AWQ_GEMM_SPLITK_STATIC_SCRATCH_BYTES,
                  "the header states the scratch size");
    awq_status st = check_layer(layer);
    if (st != AWQ_SUCCESS) return st;
    if (splits < 1 || splits > kMaxSplits) return AWQ_ERROR_INVALID_VALUE;
    st = check_io(x, y, layer, M);
    if (st != AWQ_SUCCESS || M == 0) return st;
    if (splits == 1)
        return done(stream, awq::launch_gemm(x, layer->qweight, layer->scales, layer->qzeros, y, M,
                                         layer->K, layer->N, layer->group_size, layout_of(layer), as_stream(stream)));
    if (!awq::gemm_splitk_supported(layer->K, layer->group_size, splits)) return AWQ_ERROR_UNSUPPORTED;
    if (awq::gemm_splitk_workspace(M, layer->N, splits) > awq::kStaticScratchBytes)
        return AWQ_ERROR_WORKSPACE;
    return done(stream, awq::launch_gemm_splitk_static(x, layer->qweight, layer->scales, layer->qzeros,
                                                   y, M, layer->K, layer->N, layer->group_size,
                                                   splits, layout_of(layer), as_stream(stream)));
}

size_t awq_channel_stats_workspace_bytes(int32_t M, int32_t K, int32_t N, int32_t group_size) {
    if (M <= 0 || K <= 0 || N <= 0 || group_size <= 0 || K % group_size) return 0;
    return awq::channel_stats_workspace(M, K, N, group_size);
}

size_t awq_scale_search_workspace_bytes(int32_t M, int32_t K, int32_t N, int32_t group_size) {
    if (M <= 0 || K <= 0 || N <= 0 || group_size <= 0 || K % group_size) return 0;
    return awq::scale_search_workspace(M, K, N, group_size);
}

awq_status awq_channel_stats(const uint16_t *x, int32_t M, const uint16_t *w, int32_t K, int32_t N,
                             int32_t group_size, float *xbar, float *wbar, void *workspace,
                             size_t workspace_bytes, void *stream) {
    awq_status st = check_calibration(x, M, w, K, N, group_size);
    if (st != AWQ_SUCCESS) return st;
    if (xbar == nullptr || wbar == nullptr) return AWQ_ERROR_INVALID_VALUE;
    if (workspace == nullptr || !aligned16(workspace) ||
        workspace_bytes < awq::channel_stats_workspace(M, K, N, group_size))
        return AWQ_ERROR_WORKSPACE;
    return done(stream, awq::launch_channel_stats(x, M, w, K, N, group_size, xbar, wbar, workspace,
                                              as_stream(stream)));
}

awq_status awq_scale_search(const uint16_t *x, int32_t M, const uint16_t *w, int32_t K, int32_t N,
                            int32_t group_size, int32_t symmetric, const float *alphas,
                            int32_t n_alpha, double *losses, int32_t *best, float *best_scales,
                            void *workspace, size_t workspace_bytes, void *stream) {
    awq_status st = check_calibration(x, M, w, K, N, group_size);
    if (st != AWQ_SUCCESS) return st;
    if (alphas == nullptr || losses == nullptr || best == nullptr || n_alpha < 1 ||
        n_alpha > awq::kScaleSearchMaxAlphas)
        return AWQ_ERROR_INVALID_VALUE;
    for (int i = 0; i < n_alpha; ++i)
        if (!(alphas[i] >= 0.0f && alphas[i] <= 1.0f)) return AWQ_ERROR_INVALID_VALUE;   // also NaN
    if (workspace == nullptr || !aligned16(workspace) ||
        workspace_bytes < awq::scale_search_workspace(M, K, N, group_size))
        return AWQ_ERROR_WORKSPACE;
    return done(stream, awq::launch_scale_search(x, M, w, K, N, group_size, symmetric != 0, alphas,
                                             n_alpha, losses, best, best_scales, workspace,
                                             as_stream(stream)));
}

}  // extern "C"
