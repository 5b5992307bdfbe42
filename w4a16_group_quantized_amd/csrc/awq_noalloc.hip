// Split-K GEMM on a library-owned scratch array, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): awq_gemm_splitk_static of include/awq.h.
//
// The fp32 partial tiles of the split-K GEMM go into `scratch`, a file-scope
// device array of kStaticScratchBytes that each GPU holds from the library's
// first use on it until the process ends.  In host code the array's name is
// only a host-side stand-in, so its device address is looked up once per
// device, with that device current, by hipGetSymbolAddress, and only that
// address is handed to the kernels.  Nothing in the scratch has to start at
// zero: every slice writes its whole partial tile before the reduction reads
// it.  All calls on one GPU share its array, so calls that overlap in time on
// one GPU (two streams, two host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "awq_internal.h"

namespace awq {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    hipError_t status = hipSuccess;
    void *ptr = nullptr;
};

DeviceScratch g_scratch[kMaxDevices];

// The current device's copy of `scratch` (its device address).
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        void *p = nullptr;
        d.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.status == hipSuccess) d.ptr = p;
    });
    if (d.status != hipSuccess) return d.status;
    if (d.ptr == nullptr) return hipErrorInvalidSymbol;
    *out = d.ptr;
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemm_splitk_static(const uint16_t *x, const int32_t *qweight,
                                     const uint16_t *scales, const int32_t *qzeros, uint16_t *y,
                                     int M, int K, int N, int G, int splits, int il, hipStream_t s) {
    if (gemm_splitk_workspace(M, N, splits) > kStaticScratchBytes) return hipErrorInvalidValue;
    void *ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    return launch_gemm_splitk(x, qweight, scales, qzeros, y, M, K, N, G, splits, ws, il, s);
}

}  // namespace awq
