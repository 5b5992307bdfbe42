// Timeline probe: the library's decode GEMV and batched GEMM kernels compiled
// with per-wave timestamps (AWQ_TIMELINE; the kernels are otherwise the
// library's own, from the same headers), for the accounts of where a call's
// time goes.  Each recording wave writes its start, loop end, reduction start
// (GEMV) or loop start (GEMM), end after its stores completed, and the shader
// clock at two of them, into awq_timeline[field][slot].
//   GEMV slot = workgroup * waves + wave: fields start, loop end, after the
//     workgroup barrier, end; shader clock at start and at loop end.
//   GEMM slot = workgroup (thread 0): fields start, loop start, loop end, end;
//     shader clock at loop start and at loop end.
// The kernels run in namespaces of their own (timeline_gemv, timeline_gemm),
// apart from the library's.
#define AWQ_TIMELINE 1
#define gemv timeline_gemv
#define gemm timeline_gemm
#include "../w4a16_group_quantized_amd/csrc/awq_gemv_kernels.h"
#include "../w4a16_group_quantized_amd/csrc/awq_gemm_kernels.h"

__device__ unsigned long long awq_timeline[kTimelineFields][kTimelineSlots];

namespace awq {
namespace gemm {
// The general path is not timed here.
hipError_t launch_general(const uint16_t *, const int32_t *, const uint16_t *, const int32_t *,
                          uint16_t *, int, int, int, int, int, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace gemm
}  // namespace awq
#undef gemm
#undef gemv

namespace {
hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }
}  // namespace

extern "C" {

// kind 0: the decode kernel (64-column strips, X staged up front, two segments
// in flight); kind 1: the small-batch kernel (128 columns per workgroup, as
// paired strips where N is a multiple of 16; X staged segment by segment).
// Blocked words.  Returns a hipError_t.
int awq_timeline_gemv(int kind, const void *x, const void *qw, const void *sc, const void *qz,
                      void *y, int M, int K, int N, int G, void *stream) {
    const auto *xx = static_cast<const uint16_t *>(x);
    const auto *q = static_cast<const int32_t *>(qw);
    const auto *s = static_cast<const uint16_t *>(sc);
    const auto *z = static_cast<const int32_t *>(qz);
    auto *yy = static_cast<uint16_t *>(y);
    if (kind == 0)
        return (int)awq::timeline_gemv::launch_stream_m<4, 8, 16, 2, 2>(xx, q, s, z, yy, M, K, N, G,
                                                                          as_stream(stream));
    if (kind == 1) {
        if (N % 16 == 0)   // paired strips, as the library takes them
            return (int)awq::timeline_gemv::launch_stream_prog<8, 8, 1, 2, 2>(xx, q, s, z, yy, M, K, N,
                                                                                G, as_stream(stream));
        return (int)awq::timeline_gemv::launch_stream_prog<8, 8, 1, 0, 2>(xx, q, s, z, yy, M, K, N,
                                                                            G, as_stream(stream));
    }
    return (int)hipErrorInvalidValue;
}

// awq_gemm's fast paths on blocked words.  Returns a hipError_t.
int awq_timeline_gemm(const void *x, const void *qw, const void *sc, const void *qz, void *y, int M,
                      int K, int N, int G, void *stream) {
    return (int)awq::timeline_gemm::launch_layout<2>(
        static_cast<const uint16_t *>(x), static_cast<const int32_t *>(qw),
        static_cast<const uint16_t *>(sc), static_cast<const int32_t *>(qz),
        static_cast<uint16_t *>(y), M, K, N, G, as_stream(stream));
}

// Copies the whole stamp array (fields x slots, u64) to host memory `out`.
int awq_timeline_read(unsigned long long *out) {
    return (int)hipMemcpyFromSymbol(out, HIP_SYMBOL(awq_timeline),
                                    sizeof(unsigned long long) * kTimelineFields * kTimelineSlots);
}

int awq_timeline_slots(void) { return kTimelineSlots; }

}  // extern "C"
