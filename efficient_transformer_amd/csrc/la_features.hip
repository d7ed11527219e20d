// Random-feature maps with feature dimension F (page "Stable, Fast and Accurate:
// Kernelized Attention with Relative Positional Encoding", Proposed method and
// Main findings: kernelized attention with PRF, TRF, Sphere-PRF and ORF feature
// maps, feature dimension down to 16, queries and keys normalised when their
// norms are large).  For a row x of D values and a projection W (rows w_p):
//   kind 0 (elu):  phi(x) = elu(x) + 1 elementwise, F = D, W unused;
//   kind 1 (PRF):  phi_p(x) = exp(w_p . x - |x|^2 / 2) / sqrt(F), W [F][D];
//   kind 2 (TRF):  with P = F / 2, W [P][D], c = exp(|x|^2 / 2) / sqrt(P):
//                  phi_p(x) = c sin(w_p . x), phi_{P+p}(x) = c cos(w_p . x).
// ORF and Sphere-PRF are PRF with orthogonal rows or rows on a sphere in W.
// NORM: every row is scaled to unit length first.
//
// One workgroup maps 64 rows: the 64 x D tile is staged in LDS with coalesced
// 16-byte loads, each lane then owns one row, and each of the 4 wavefronts
// forms a quarter of the projections.  W is read with wave-uniform addresses
// (scalar loads), so every fma takes its W operand from a scalar register.  The
// 64 x F results go back through LDS and leave as coalesced 16-byte stores.
// The projection is a dense contraction, but on gfx950 fp32 matrix and fp32
// vector throughput are the same (157.3 TFLOP/s), and at F = 16 the kernel is
// bound by HBM: vector fmas with scalar operands need no operand shuffling.
#include <math.h>

#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

constexpr int kFeatRows = 64;
constexpr int kFeatThreads = 256;

template <int D, int F, int KIND>
struct FeatCfg {
    static constexpr int P = KIND == 2 ? F / 2 : F;  // projections (kind 0: columns)
    static constexpr int PW = P / 4;                 // per wavefront
    static constexpr int LX = D + 4;                 // LDS row of the input tile (floats)
    static constexpr int LO = F + 4;                 // LDS row of the output tile
    static_assert(PW >= 1 && PW * 4 == P, "projections split over 4 wavefronts");
};

template <typename T>
__device__ __forceinline__ f32x4 feat_load4(const T *p);
template <>
__device__ __forceinline__ f32x4 feat_load4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <>
__device__ __forceinline__ f32x4 feat_load4<bf16>(const bf16 *p) {
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

// blockIdx.y selects the tensor: 0 -> (X, out), 1 -> (X2, out2).
template <typename T, int D, int F, int KIND, bool NORM>
__global__ __launch_bounds__(kFeatThreads) void feature_map_kernel(const T *__restrict__ X, float *__restrict__ out,
                                                                   const T *__restrict__ X2, float *__restrict__ out2,
                                                                   const float *__restrict__ W, long rows) {
    using G = FeatCfg<D, F, KIND>;
    __shared__ __attribute__((aligned(16))) float sx[kFeatRows * G::LX];
    __shared__ __attribute__((aligned(16))) float so[kFeatRows * G::LO];
    const T *Xs = blockIdx.y == 0 ? X : X2;
    float *Os = blockIdx.y == 0 ? out : out2;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long r0 = (long)blockIdx.x * kFeatRows;
    const int nr = (int)(rows - r0 < kFeatRows ? rows - r0 : kFeatRows);

    // 1. the input tile; rows past the end are zero (their results are not stored)
    constexpr int V4 = D / 4;
#pragma unroll
    for (int e = tid; e < kFeatRows * V4; e += kFeatThreads) {
        const int r = e / V4, c = (e % V4) * 4;
        f32x4 v = zero4();
        if (r < nr) v = feat_load4<T>(Xs + (size_t)(r0 + r) * D + c);
        *reinterpret_cast<f32x4 *>(sx + r * G::LX + c) = v;
    }
    __syncthreads();

    // 2. lane = row: |x|^2 (and the normalising scale), then this wavefront's projections
    const float *xr = sx + lane * G::LX;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + c);
        sq += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    float scale = 1.0f;
    if (NORM && sq > 0.0f) {
        scale = 1.0f / sqrtf(sq);
        sq = sq * scale * scale;
    }
    float *orow = so + lane * G::LO;
    if constexpr (KIND == 0) {
#pragma unroll
        for (int j = 0; j < G::PW; ++j) {
            const int col = w * G::PW + j;
            orow[col] = phi(xr[col] * scale);
        }
    } else {
        float acc[G::PW];
#pragma unroll
        for (int j = 0; j < G::PW; ++j) acc[j] = 0.0f;
        const float *Wb = W + (size_t)(w * G::PW) * D;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + c);
#pragma unroll
            for (int j = 0; j < G::PW; ++j) {
                const float *wp = Wb + (size_t)j * D + c;
                acc[j] += v[0] * wp[0] + v[1] * wp[1] + v[2] * wp[2] + v[3] * wp[3];
            }
        }
        if constexpr (KIND == 1) {
            const float inv = 1.0f / sqrtf((float)F);
#pragma unroll
            for (int j = 0; j < G::PW; ++j) orow[w * G::PW + j] = __expf(acc[j] * scale - 0.5f * sq) * inv;
        } else {
            const float c = __expf(0.5f * sq) / sqrtf((float)G::P);
#pragma unroll
            for (int j = 0; j < G::PW; ++j) {
                float s, co;
                sincosf(acc[j] * scale, &s, &co);
                orow[w * G::PW + j] = c * s;
                orow[G::P + w * G::PW + j] = c * co;
            }
        }
    }
    __syncthreads();

    // 3. coalesced stores of the valid rows
    constexpr int O4 = F / 4;
#pragma unroll
    for (int e = tid; e < kFeatRows * O4; e += kFeatThreads) {
        const int r = e / O4, c = (e % O4) * 4;
        if (r < nr)
            *reinterpret_cast<f32x4 *>(Os + (size_t)(r0 + r) * F + c) =
                *reinterpret_cast<const f32x4 *>(so + r * G::LO + c);
    }
}

template <typename T, int D, int F, int KIND>
hipError_t run_feature_map(const void *X, float *out, const void *X2, float *out2, const float *W, long rows,
                           bool norm, hipStream_t stream) {
    if constexpr (KIND == 0 && D != F) {
        return hipErrorInvalidValue;  // the elementwise map keeps the width
    } else {
        if (rows <= 0) return hipSuccess;
        const dim3 grid((unsigned)((rows + kFeatRows - 1) / kFeatRows), X2 != nullptr ? 2u : 1u);
        if (norm)
            hipLaunchKernelGGL((feature_map_kernel<T, D, F, KIND, true>), grid, dim3(kFeatThreads), 0, stream,
                               (const T *)X, out, (const T *)X2, out2, W, rows);
        else
            hipLaunchKernelGGL((feature_map_kernel<T, D, F, KIND, false>), grid, dim3(kFeatThreads), 0, stream,
                               (const T *)X, out, (const T *)X2, out2, W, rows);
        return hipGetLastError();
    }
}

template <typename T>
hipError_t feature_map_t(int D, int F, int kind, const void *X, float *out, const void *X2, float *out2,
                         const float *W, long rows, bool norm, hipStream_t stream) {
#define X_(D_, F_)                                                                                        \
    if (D == D_ && F == F_) {                                                                             \
        if (kind == 1) return run_feature_map<T, D_, F_, 1>(X, out, X2, out2, W, rows, norm, stream);      \
        if (kind == 2) return run_feature_map<T, D_, F_, 2>(X, out, X2, out2, W, rows, norm, stream);      \
        if (kind == 0) return run_feature_map<T, D_, F_, 0>(X, out, X2, out2, W, rows, norm, stream);      \
    }
#define XF_(D_) X_(D_, 16) X_(D_, 32) X_(D_, 64) X_(D_, 128)
    XF_(16) XF_(32) XF_(64) XF_(128)
#undef XF_
#undef X_
    return hipErrorInvalidValue;
}

hipError_t feature_map(int dtype, int D, int F, int kind, const void *X, float *out, const void *X2, float *out2,
                       const float *W, long rows, bool norm, hipStream_t stream) {
    return dtype == kDtypeBf16 ? feature_map_t<bf16>(D, F, kind, X, out, X2, out2, W, rows, norm, stream)
                               : feature_map_t<float>(D, F, kind, X, out, X2, out2, W, rows, norm, stream);
}

}  // namespace la
