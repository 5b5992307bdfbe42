// AWQ's scale search: per-input-channel statistics of calibration activations
// and weights, candidate scales c, the migrated layer (X / c, c W) quantized and
// multiplied by the fused GEMM, and its output error against the fp16 layer
// (pyshine.com AutoAWQ tour, "The Quantization Flow Up Close": the per-channel
// mean of normalized weights and the mean of activations, the FP16 module run
// once as the reference, the candidate of least output error; scale_ln_fcs:
// dividing the preceding op's output by c and multiplying the weights by c is
// invisible before rounding).  The pages give neither the normalization, the
// candidate formula nor the grid; the readings taken:
//   xbar[k] = mean over rows of |x(m, k)|;
//   wbar[k] = mean over columns n of |w(k, n)| / a(g, n), a(g, n) the largest
//             |w| of k's quantization group in column n (0 if a = 0);
//   c[k]    = max(xbar, 1e-4)^alpha / max(wbar, 1e-4)^(1 - alpha), alpha from
//             the caller's grid;
//   loss    = mean over (m, n) of (y - y')^2, y = X W in fp32 (MFMA), y' the
//             fused GEMM's fp16 output for fp16(X / c) and the quantized
//             fp16(c W); the first alpha of least loss is kept.
// All reductions run in a fixed order (fp64 partial sums), so a loss is the
// same bits on every run.  The search is calibration work, done once per layer:
// the kernels here are plain, and the time goes to the quantizer and the fused
// GEMM of each candidate, which are the layer's own kernels.  The quantizer
// forms fp16(c W) row by row as it reads W, so no migrated weight is written.
#include "awq_device.h"
#include "awq_internal.h"

namespace awq {
namespace scale {

constexpr int kStatRows = 64;       // calibration rows per partial-sum chunk of xbar, at least
constexpr int kStatCols = 512;      // columns per xbar block (64 lanes x 8)
constexpr int kLossBlocks = 1024;   // blocks of the squared-error reduction
constexpr float kFloor = 1e-4f;

__device__ __forceinline__ void halves8(uint4 v, float f[8]) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = (float)as_half((uint16_t)u[i]);
        f[2 * i + 1] = (float)as_half((uint16_t)(u[i] >> 16));
    }
}

__device__ __forceinline__ uint4 pack8(const float f[8]) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        u[i] = (uint32_t)as_u16((half_t)f[2 * i]) | ((uint32_t)as_u16((half_t)f[2 * i + 1]) << 16);
    return make_uint4(u[0], u[1], u[2], u[3]);
}

// Sum of a double over the block (blockDim.x a power of two up to 256), in a
// fixed tree order; the result is valid in thread 0.
__device__ __forceinline__ double block_sum(double v, double *sh) {
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int o = blockDim.x / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
        __syncthreads();
    }
    return sh[0];
}

// Rows per xbar chunk: kStatRows, or more when M would need more than 65535
// chunks (the grid's y limit).
inline int stat_rows(int M) { return max(kStatRows, (M + 65534) / 65535); }

// xbar, pass 1: partial[chunk][k] = sum of |x(m, k)| over the chunk's rows.
// Block (column block b, chunk r): 64 lanes x 8 columns, `rows` rows.
__global__ void __launch_bounds__(64)
act_partial_kernel(const uint16_t *__restrict__ X, int M, int K, int rows,
                   double *__restrict__ partial) {
    const int k0 = blockIdx.x * kStatCols + 8 * threadIdx.x;
    if (k0 >= K) return;
    const int r0 = blockIdx.y * rows, r1 = min(M, r0 + rows);
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int m = r0; m < r1; ++m) {
        float f[8];
        halves8(*reinterpret_cast<const uint4 *>(X + (size_t)m * K + k0), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += fabsf(f[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) partial[(size_t)blockIdx.y * K + k0 + i] = acc[i];
}

// xbar, pass 2: the chunks in order, divided by M.
__global__ void act_final_kernel(const double *__restrict__ partial, int chunks, int M, int K,
                                 float *__restrict__ xbar) {
    for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < K; k += gridDim.x * blockDim.x) {
        double s = 0.0;
        for (int r = 0; r < chunks; ++r) s += partial[(size_t)r * K + k];
        xbar[k] = (float)(s / M);
    }
}

// a(g, n) = max |w| over group g of column n, for 8 columns per thread.
__global__ void group_absmax_kernel(const uint16_t *__restrict__ W, int K, int N, int G,
                                    float *__restrict__ A) {
    const long long total = (long long)(K / G) * (N / 8);
    for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const int g = (int)(t / (N / 8)), n = (int)(t % (N / 8)) * 8;
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int k = g * G; k < (g + 1) * G; ++k) {
            float f[8];
            halves8(*reinterpret_cast<const uint4 *>(W + (size_t)k * N + n), f);
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = fmaxf(a[i], fabsf(f[i]));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) A[(size_t)g * N + n + i] = a[i];
    }
}

// wbar[k] = mean over n of |w(k, n)| / a(g, n): one block of 256 threads per row.
__global__ void __launch_bounds__(256)
wbar_kernel(const uint16_t *__restrict__ W, const float *__restrict__ A, int K, int N, int G,
            float *__restrict__ wbar) {
    __shared__ double sh[256];
    const int k = blockIdx.x;
    const uint16_t *row = W + (size_t)k * N;
    const float *arow = A + (size_t)(k / G) * N;
    double acc = 0.0;
    for (int n = 8 * threadIdx.x; n < N; n += 8 * 256) {
        float f[8];
        halves8(*reinterpret_cast<const uint4 *>(row + n), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float a = arow[n + i];
            if (a > 0.0f) acc += fabsf(f[i]) / a;
        }
    }
    const double s = block_sum(acc, sh);
    if (threadIdx.x == 0) wbar[k] = (float)(s / N);
}

__device__ __forceinline__ float candidate(float xb, float wb, float alpha) {
    return powf(fmaxf(xb, kFloor), alpha) / powf(fmaxf(wb, kFloor), 1.0f - alpha);
}

__global__ void candidate_kernel(const float *__restrict__ xbar, const float *__restrict__ wbar,
                                 int K, float alpha, float *__restrict__ c) {
    for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < K; k += gridDim.x * blockDim.x)
        c[k] = candidate(xbar[k], wbar[k], alpha);
}

// X'(m, k) = fp16(x / c[k]), 8 values per thread.
__global__ void migrate_x_kernel(const uint16_t *__restrict__ X, const float *__restrict__ c, int M,
                                 int K, uint16_t *__restrict__ Xs) {
    const long long total = (long long)M * K / 8;
    for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const int k0 = (int)((t * 8) % K);   // a multiple of 8: c + k0 is 32-byte aligned
        const float4 c0 = reinterpret_cast<const float4 *>(c + k0)[0];
        const float4 c1 = reinterpret_cast<const float4 *>(c + k0)[1];
        const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        float f[8];
        halves8(reinterpret_cast<const uint4 *>(X)[t], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = f[i] / cv[i];
        reinterpret_cast<uint4 *>(Xs)[t] = pack8(f);
    }
}

// The fp16 layer's output y = X W in fp32, for the reference: a 128 x 128 tile
// per workgroup (a 1-D grid, tile rows minor), four waves of 2 x 2
// v_mfma_f32_32x32x16_f16 tiles each, 32-k steps through a two-slot LDS ring
// (the next step's loads are in flight during the MFMAs; one barrier a step).
// W is stored transposed, [n][k], so that a lane's B operand (8 k of one
// column) is one 16-byte read: each lane loads 8 consecutive k of one column
// (2-byte loads, coalesced along n across the lanes) and writes them as one
// 16-byte chunk.  Rows past M, columns past N and k past K load zeros and are
// not stored.
constexpr int kDT = 128, kDK = 32, kDPad = kDK + 8;   // row stride 40 halves: 80 bytes

__global__ void __launch_bounds__(256)
dense_gemm_kernel(const uint16_t *__restrict__ X, const uint16_t *__restrict__ W, int M, int K,
                  int N, float *__restrict__ Y) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kDT][kDPad];
    __shared__ __attribute__((aligned(16))) uint16_t Bt[2][kDT][kDPad];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int tiles_m = (M + kDT - 1) / kDT;
    const int m0 = (int)(blockIdx.x % tiles_m) * kDT, n0 = (int)(blockIdx.x / tiles_m) * kDT;
    const int wr = 64 * (wave >> 1), wc = 64 * (wave & 1);
    // Chunk i (0, 1) of this thread: X row c / 4, k offset 8 (c % 4); W column
    // c % 128, k octet c / 128; with c = t + 256 i.
    uint4 ra[2], rb[2];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = t + 256 * i;
            const int row = c >> 2, kc = (c & 3) * 8;
            ra[i] = (m0 + row < M && k0 + kc < K)
                        ? *reinterpret_cast<const uint4 *>(X + (size_t)(m0 + row) * K + k0 + kc)
                        : make_uint4(0u, 0u, 0u, 0u);
            const int n = c & (kDT - 1), k8 = k0 + 8 * (c >> 7);
            uint32_t h[4] = {0u, 0u, 0u, 0u};
            if (k8 < K && n0 + n < N) {
                const uint16_t *wp = W + (size_t)k8 * N + n0 + n;
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e / 2] |= (uint32_t)wp[(size_t)e * N] << (16 * (e % 2));
            }
            rb[i] = make_uint4(h[0], h[1], h[2], h[3]);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = t + 256 * i;
            *reinterpret_cast<uint4 *>(&As[buf][c >> 2][(c & 3) * 8]) = ra[i];
            *reinterpret_cast<uint4 *>(&Bt[buf][c & (kDT - 1)][8 * (c >> 7)]) = rb[i];
        }
    };
    float16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    gload(0);
    sstore(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < K; k0 += kDK) {
        const bool more = k0 + kDK < K;
        if (more) gload(k0 + kDK);
#pragma unroll
        for (int kk = 0; kk < kDK; kk += 16) {
            const int kl = kk + 8 * (lane >> 5);
            half8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = as_half8(*reinterpret_cast<const uint4 *>(&As[buf][wr + 32 * i + (lane & 31)][kl]));
                b[i] = as_half8(*reinterpret_cast<const uint4 *>(&Bt[buf][wc + 32 * i + (lane & 31)][kl]));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        // The other slot was last read in the previous step, before its barrier.
        if (more) sstore(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    // C layout: lane (h, j) holds in register v row 8 (v / 4) + 4 h + v % 4 of column j.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + wc + 32 * j + (lane & 31);
        if (col >= N) continue;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wr + 32 * i + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
                if (row < M) Y[(size_t)row * N + col] = acc[i][j][v];
            }
    }
}

// Squared error of the candidate's fp16 output against the fp32 reference:
// per-block fp64 partial sums over a grid-stride range.
__global__ void __launch_bounds__(256)
sqerr_kernel(const float *__restrict__ Yref, const uint16_t *__restrict__ Yhat, long long count,
             double *__restrict__ partial) {
    // Eight outputs per lane and iteration (count = M N is a multiple of 8, both
    // arrays 16-byte aligned): two 16-byte loads of Yref and one of Yhat.
    __shared__ double sh[256];
    double acc = 0.0;
    const long long n8 = count / 8;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const f32x4 *yr = reinterpret_cast<const f32x4 *>(Yref);
    const u32x4 *yh = reinterpret_cast<const u32x4 *>(Yhat);
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n8; i += (long long)gridDim.x * 256) {
        const f32x4 a = __builtin_nontemporal_load(yr + 2 * i);
        const f32x4 b = __builtin_nontemporal_load(yr + 2 * i + 1);
        const u32x4 h = __builtin_nontemporal_load(yh + i);
        float f[8];
        halves8(make_uint4(h.x, h.y, h.z, h.w), f);
        const float r[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double d = (double)r[e] - (double)f[e];
            acc += d * d;
        }
    }
    const double s = block_sum(acc, sh);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

__global__ void __launch_bounds__(256)
loss_final_kernel(const double *__restrict__ partial, int blocks, long long count,
                  double *__restrict__ loss) {
    __shared__ double sh[256];
    double acc = 0.0;
    for (int b = threadIdx.x; b < blocks; b += 256) acc += partial[b];
    const double s = block_sum(acc, sh);
    if (threadIdx.x == 0) *loss = s / (double)count;
}

struct Alphas {
    float a[kScaleSearchMaxAlphas];
};

// The first alpha of least loss, and (optionally) its scales.
__global__ void __launch_bounds__(256)
argmin_kernel(const double *__restrict__ losses, int n, Alphas alphas, const float *__restrict__ xbar,
              const float *__restrict__ wbar, int K, int32_t *__restrict__ best,
              float *__restrict__ best_scales) {
    __shared__ int bi;
    if (threadIdx.x == 0) {
        int b = 0;
        for (int i = 1; i < n; ++i)
            if (losses[i] < losses[b]) b = i;
        bi = b;
        *best = b;
    }
    __syncthreads();
    if (best_scales == nullptr) return;
    const float alpha = alphas.a[bi];
    for (int k = threadIdx.x; k < K; k += 256) best_scales[k] = candidate(xbar[k], wbar[k], alpha);
}

// Workspace regions, each 256-byte aligned.
struct Layout {
    size_t act, amax, xbar, wbar, c, xs, q, s, qz, yref, yhat, loss, total;
};

inline size_t up256(size_t b) { return (b + 255) & ~size_t(255); }

Layout layout(int M, int K, int N, int G, bool search) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += up256(bytes);
        return o;
    };
    const size_t chunks = (size_t)(M + stat_rows(M) - 1) / stat_rows(M);
    L.act = take(chunks * K * sizeof(double));
    L.amax = take((size_t)(K / G) * N * sizeof(float));
    if (search) {
        L.xbar = take((size_t)K * sizeof(float));
        L.wbar = take((size_t)K * sizeof(float));
        L.c = take((size_t)K * sizeof(float));
        L.xs = take((size_t)M * K * 2);
        L.q = take((size_t)K / 8 * N * 4);
        L.s = take((size_t)(K / G) * N * 2);
        L.qz = take((size_t)(K / G) * (N / 8) * 4);
        L.yref = take((size_t)M * N * sizeof(float));
        L.yhat = take((size_t)M * N * 2);
        L.loss = take(kLossBlocks * sizeof(double));
    }
    L.total = off;
    return L;
}

inline unsigned grid_for(long long items, int per_block) {
    const long long b = (items + per_block - 1) / per_block;
    return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

hipError_t stats(const uint16_t *x, int M, const uint16_t *w, int K, int N, int G, float *xbar,
                 float *wbar, char *ws, const Layout &L, hipStream_t s) {
    auto *act = reinterpret_cast<double *>(ws + L.act);
    auto *amax = reinterpret_cast<float *>(ws + L.amax);
    const int rows = stat_rows(M), chunks = (M + rows - 1) / rows;
    hipLaunchKernelGGL(act_partial_kernel, dim3((K + kStatCols - 1) / kStatCols, chunks), dim3(64), 0,
                       s, x, M, K, rows, act);
    hipLaunchKernelGGL(act_final_kernel, dim3(grid_for(K, 256)), dim3(256), 0, s, act, chunks, M, K,
                       xbar);
    hipLaunchKernelGGL(group_absmax_kernel, dim3(grid_for((long long)(K / G) * (N / 8), 256)),
                       dim3(256), 0, s, w, K, N, G, amax);
    hipLaunchKernelGGL(wbar_kernel, dim3(K), dim3(256), 0, s, w, amax, K, N, G, wbar);
    return hipGetLastError();
}

}  // namespace scale

size_t channel_stats_workspace(int M, int K, int N, int G) {
    return scale::layout(M, K, N, G, false).total;
}

size_t scale_search_workspace(int M, int K, int N, int G) {
    return scale::layout(M, K, N, G, true).total;
}

hipError_t launch_channel_stats(const uint16_t *x, int M, const uint16_t *w, int K, int N, int G,
                                float *xbar, float *wbar, void *workspace, hipStream_t s) {
    const scale::Layout L = scale::layout(M, K, N, G, false);
    return scale::stats(x, M, w, K, N, G, xbar, wbar, static_cast<char *>(workspace), L, s);
}

hipError_t launch_scale_search(const uint16_t *x, int M, const uint16_t *w, int K, int N, int G,
                               bool symmetric, const float *alphas, int n_alpha, double *losses,
                               int32_t *best, float *best_scales, void *workspace, hipStream_t s) {
    using namespace scale;
    const Layout L = layout(M, K, N, G, true);
    char *ws = static_cast<char *>(workspace);
    auto *xbar = reinterpret_cast<float *>(ws + L.xbar);
    auto *wbar = reinterpret_cast<float *>(ws + L.wbar);
    auto *c = reinterpret_cast<float *>(ws + L.c);
    auto *xs = reinterpret_cast<uint16_t *>(ws + L.xs);
    auto *q = reinterpret_cast<int32_t *>(ws + L.q);
    auto *sc = reinterpret_cast<uint16_t *>(ws + L.s);
    auto *qz = symmetric ? nullptr : reinterpret_cast<int32_t *>(ws + L.qz);
    auto *yref = reinterpret_cast<float *>(ws + L.yref);
    auto *yhat = reinterpret_cast<uint16_t *>(ws + L.yhat);
    auto *part = reinterpret_cast<double *>(ws + L.loss);
    const long long mn = (long long)M * N;

    hipError_t e = stats(x, M, w, K, N, G, xbar, wbar, ws, L, s);
    if (e != hipSuccess) return e;
    const long long dtiles = (long long)((M + kDT - 1) / kDT) * ((N + kDT - 1) / kDT);
    hipLaunchKernelGGL(dense_gemm_kernel, dim3((unsigned)dtiles), dim3(256), 0, s, x, w, M, K, N, yref);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    for (int i = 0; i < n_alpha; ++i) {
        hipLaunchKernelGGL(candidate_kernel, dim3(grid_for(K, 256)), dim3(256), 0, s, xbar, wbar, K,
                           alphas[i], c);
        hipLaunchKernelGGL(migrate_x_kernel, dim3(grid_for((long long)M * K / 8, 256)), dim3(256), 0,
                           s, x, c, M, K, xs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // the migrated weight fp16(c W) is formed row by row inside the quantizer
        if ((e = launch_quantize_migrated(w, c, q, sc, qz, K, N, G, symmetric, s)) != hipSuccess)
            return e;
        if ((e = launch_gemm(xs, q, sc, qz, yhat, M, K, N, G, 0 /* canonical words */, s)) != hipSuccess) return e;
        hipLaunchKernelGGL(sqerr_kernel, dim3(kLossBlocks), dim3(256), 0, s, yref, yhat, mn, part);
        hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(256), 0, s, part, kLossBlocks, mn,
                           losses + i);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    Alphas a{};
    for (int i = 0; i < n_alpha; ++i) a.a[i] = alphas[i];
    hipLaunchKernelGGL(argmin_kernel, dim3(1), dim3(256), 0, s, losses, n_alpha, a, xbar, wbar, K, best,
                       best_scales);
    return hipGetLastError();
}

}  // namespace awq
