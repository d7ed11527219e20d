// Peak probes: the attainable rates that the kernels' rooflines are set against.
//   la_probe_copy: a plain device-to-device copy (16-byte words, four in flight
//                  per thread) -> attainable HBM read + write rate;
//   la_probe_mfma: chains of fp32 16x16x4 or bf16 16x16x32 MFMAs on eight
//                  independent accumulators per wavefront -> attainable matrix rate.
// Both are checkable: the copy is bit-exact and every MFMA chain reaches a value
// known in closed form (see la_probe_mfma in include/linattn.h).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "la_device.hpp"
#include "linattn.h"

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int kMfmaThreads = 256;
constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(kCopyThreads) void probe_copy_kernel(const la::f32x4 *__restrict__ src,
                                                                  la::f32x4 *__restrict__ dst, size_t n4) {
    const size_t step = (size_t)gridDim.x * kCopyThreads * kCopyUnroll;
    for (size_t i = (size_t)blockIdx.x * kCopyThreads * kCopyUnroll + threadIdx.x; i < n4; i += step) {
        la::f32x4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t j = i + (size_t)u * kCopyThreads;
            if (j < n4) v[u] = src[j];
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t j = i + (size_t)u * kCopyThreads;
            if (j < n4) dst[j] = v[u];
        }
    }
}

// Every operand element is x (rounded to the operand type); each MFMA adds K x^2
// to every accumulator element.  Each lane writes the sum of its 32 accumulator
// values.
template <bool BF16>
__global__ __launch_bounds__(kMfmaThreads) void probe_mfma_kernel(float *__restrict__ out, int iters, float x) {
    la::f32x4 c[kMfmaChains];
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) c[j] = la::zero4();
    if constexpr (BF16) {
        const la::bf16 h = (la::bf16)x;
        const la::bf16x8 a = {h, h, h, h, h, h, h, h};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kMfmaChains; ++j) c[j] = la::mma_bf16_k32(a, a, c[j]);
        }
    } else {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kMfmaChains; ++j) c[j] = la::mma_f32(x, x, c[j]);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) s += (c[j][0] + c[j][1]) + (c[j][2] + c[j][3]);
    out[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

int status_of(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_HIP; }

}  // namespace

extern "C" {

LA_API int la_probe_copy(void *dst, const void *src, size_t bytes, void *stream) {
    if (bytes % 16 != 0) return LA_ERR_INVALID_ARG;
    if (bytes == 0) return LA_OK;
    if (!dst || !src || ((uintptr_t)dst & 15u) || ((uintptr_t)src & 15u)) return LA_ERR_INVALID_ARG;
    const size_t n4 = bytes / 16;
    const size_t per_block = (size_t)kCopyThreads * kCopyUnroll;
    // enough workgroups to fill every CU many times over; the loop strides over the rest
    const size_t blocks = std::min<size_t>((n4 + per_block - 1) / per_block, 256 * 16);
    (void)hipGetLastError();
    hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const la::f32x4 *>(src),
                       static_cast<la::f32x4 *>(dst), n4);
    return status_of(hipGetLastError());
}

LA_API int la_probe_mfma(float *out, int dtype, int64_t blocks, int iters, float x, void *stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
    if (blocks < 0 || blocks > (1 << 20) || iters < 0) return LA_ERR_INVALID_ARG;
    if (blocks == 0) return LA_OK;
    if (!out) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == LA_BF16)
        hipLaunchKernelGGL(probe_mfma_kernel<true>, dim3((unsigned)blocks), dim3(kMfmaThreads), 0, s, out, iters, x);
    else
        hipLaunchKernelGGL(probe_mfma_kernel<false>, dim3((unsigned)blocks), dim3(kMfmaThreads), 0, s, out, iters, x);
    return status_of(hipGetLastError());
}

}  // extern "C"
