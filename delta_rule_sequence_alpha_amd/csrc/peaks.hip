// Reference kernels for measured machine peaks (include/efla_peaks.h): a
// streaming copy for HBM bandwidth and MFMA loops for matrix-core throughput.
// They compute nothing of the operator; bench.py states every roofline
// fraction against the published peaks and against what these reach.
#include <stdint.h>

#include "efla_device.h"
#include "efla_peaks.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Each thread moves UNROLL 16-byte vectors per stride step, all loads issued
// before the stores; the grid strides over the buffer.
constexpr int kCopyThreads = 256, kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const u32x4 *__restrict__ src,
                                                            u32x4 *__restrict__ dst, long n)
{
    const long stride = (long)gridDim.x * kCopyThreads * kCopyUnroll;
    for (long base = (long)blockIdx.x * kCopyThreads * kCopyUnroll + threadIdx.x; base < n;
         base += stride) {
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const long i = base + (long)u * kCopyThreads;
            if (i < n) v[u] = src[i];
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const long i = base + (long)u * kCopyThreads;
            if (i < n) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

// Eight independent accumulators per wave, operands fixed in registers:
// the MFMA pipe's issue rate bounds the loop.  (Left at the default launch
// bound: with the register budget of a 256-thread bound the compiler rotates
// the accumulators through copies inside the loop.)
__global__ void mfma_bf16_kernel(float *sink, int iters)
{
    const int lane = threadIdx.x & 63;
    efla::bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(1e-3f * (lane + i));
        b[i] = static_cast<__bf16>(1e-3f * (i - lane));
    }
    efla::f32x4 acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = efla::f32x4{0.f, 0.f, 0.f, static_cast<float>(n)};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[n] = efla::mma(a, b, acc[n]);
    float s = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) s += acc[n][0] + acc[n][3];
    if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

__global__ void mfma_f32_kernel(float *sink, int iters)
{
    const int lane = threadIdx.x & 63;
    const float a = 1e-3f * lane, b = 1e-3f * (3 - lane);
    efla::f32x4 acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = efla::f32x4{0.f, 0.f, 0.f, static_cast<float>(n)};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[n] = efla::mma(a, b, acc[n]);
    float s = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) s += acc[n][0] + acc[n][3];
    if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

efla_status_t efla_peak_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes % 16 != 0)
        return EFLA_ERR_INVALID_ARG;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (bytes > 0 && s < d + bytes && d < s + bytes) return EFLA_ERR_INVALID_ARG;
    if (bytes == 0) return EFLA_OK;
    const long n = (long)(bytes / 16);
    const long per_block = (long)kCopyThreads * kCopyUnroll;
    long blocks = (n + per_block - 1) / per_block;
    if (blocks > 256 * 8) blocks = 256 * 8;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src),
                       static_cast<u32x4 *>(dst), n);
    return hipGetLastError() == hipSuccess ? EFLA_OK : EFLA_ERR_HIP;
}

efla_status_t efla_peak_mfma(float *sink, int blocks, int iters, efla_dtype_t dt, double *flops,
                             void *stream)
{
    if (!sink || blocks < 1 || iters < 1 || (dt != EFLA_BF16 && dt != EFLA_F32))
        return EFLA_ERR_INVALID_ARG;
    const double per_mfma = dt == EFLA_BF16 ? 16.0 * 16 * 32 * 2 : 16.0 * 16 * 4 * 2;
    if (flops) *flops = per_mfma * 8.0 * iters * 4.0 * blocks;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dt == EFLA_BF16)
        hipLaunchKernelGGL(mfma_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, sink, iters);
    else
        hipLaunchKernelGGL(mfma_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, sink, iters);
    return hipGetLastError() == hipSuccess ? EFLA_OK : EFLA_ERR_HIP;
}

}  // extern "C"
