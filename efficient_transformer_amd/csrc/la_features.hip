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
// One workgroup maps 64 rows: the 64 x D tile and W are staged in LDS with
// coalesced 16-byte loads.  The projection x W^T is a dense contraction and runs
// on fp32 MFMA (16x16x4): each wavefront takes 16 rows, and per 16-deep block
// one 16-byte LDS read of x and one of each 16-row W tile feed four MFMAs (a
// lane-per-row vector-fma form needed an LDS read per four fmas and was
// LDS-bound beyond F = 16).  The 64 x F results go back through LDS and leave
// as coalesced 16-byte stores.
#include <math.h>

#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

constexpr int kFeatRows = 64;
constexpr int kFeatThreads = 256;

template <int D, int F, int KIND>
struct FeatCfg {
    static constexpr int P = KIND == 2 ? F / 2 : F;  // projections (kind 0: columns)
    static constexpr int PW = P / 4;                 // kind 0: columns per wavefront
    static constexpr int PT = (P + 15) / 16;         // 16-wide projection tiles (W rows past P are zero)
    static constexpr int LX = D + 4;                 // LDS row of the input tile (floats)
    static constexpr int LW = D + 4;                 // LDS row of W
    static constexpr int LO = F + 4;                 // LDS row of the output tile
    static_assert(PW >= 1 && PW * 4 == P, "projections split over 4 wavefronts");
    static_assert(D % 16 == 0 && P % 4 == 0, "16-deep contraction blocks, 4-wide result groups");
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
__global__ __launch_bounds__(kFeatThreads, 2) void feature_map_kernel(const T *__restrict__ X, float *__restrict__ out,
                                                                   const T *__restrict__ X2, float *__restrict__ out2,
                                                                   const float *__restrict__ W, long rows) {
    using G = FeatCfg<D, F, KIND>;
    __shared__ __attribute__((aligned(16))) float sx[kFeatRows * G::LX];
    __shared__ __attribute__((aligned(16))) float so[kFeatRows * G::LO];
    __shared__ __attribute__((aligned(16))) float sw[KIND == 0 ? 4 : G::PT * 16 * G::LW];  // W (padded rows)
    const T *Xs = blockIdx.y == 0 ? X : X2;
    float *Os = blockIdx.y == 0 ? out : out2;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long r0 = (long)blockIdx.x * kFeatRows;
    const int nr = (int)(rows - r0 < kFeatRows ? rows - r0 : kFeatRows);

    // 1. the input tile and W: every load issued before the first LDS write (rows
    //    past the end reload the last row; their results are not stored)
    constexpr int V4 = D / 4;
    constexpr int NL = kFeatRows * V4 / kFeatThreads;
    constexpr int WL = KIND == 0 ? 0 : (G::PT * 16 * D / 4 + kFeatThreads - 1) / kFeatThreads;
    static_assert(NL * kFeatThreads == kFeatRows * V4, "whole tile per pass");
    f32x4 xv[NL], wv[WL > 0 ? WL : 1];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = tid + i * kFeatThreads, r = e / V4, c = (e % V4) * 4;
        xv[i] = feat_load4<T>(Xs + (size_t)(r0 + min(r, nr - 1)) * D + c);
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
        const int e = min(tid + i * kFeatThreads, G::P * D / 4 - 1);  // rows past P: zero below
        wv[i] = *reinterpret_cast<const f32x4 *>(W + (size_t)e * 4);
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e = tid + i * kFeatThreads, r = e / V4, c = (e % V4) * 4;
        *reinterpret_cast<f32x4 *>(sx + r * G::LX + c) = xv[i];
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
        const int e = tid + i * kFeatThreads, f = e / (D / 4), c = (e % (D / 4)) * 4;
        if (f < G::PT * 16) *reinterpret_cast<f32x4 *>(sw + f * G::LW + c) = f < G::P ? wv[i] : zero4();
    }
    __syncthreads();

    if constexpr (KIND == 0) {
        // 2. elementwise: lane = row, wavefront w takes a quarter of the columns
        const float *xr = sx + lane * G::LX;
        float sq = 0.0f;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
            const f32x4 x4 = *reinterpret_cast<const f32x4 *>(xr + c);
            sq += x4[0] * x4[0] + x4[1] * x4[1] + x4[2] * x4[2] + x4[3] * x4[3];
        }
        const float scale = NORM && sq > 0.0f ? 1.0f / sqrtf(sq) : 1.0f;
#pragma unroll
        for (int j = 0; j < G::PW; ++j) {
            const int col = w * G::PW + j;
            so[lane * G::LO + col] = phi(xr[col] * scale);
        }
    } else {
        // 2. projections on MFMA: wavefront w owns rows 16w .. 16w+15 of the tile.
        //    C[f][row] = sum_k W[f][k] x[row][k] with W as the A operand (lane: row
        //    f = l16 of a 16-row W tile) and x as the B operand (lane: row l16 of the
        //    wavefront's rows); lane (g, l16) ends with projections 4g .. 4g+3 of its
        //    own row l16.  Within each 16-deep block, lane g contracts over
        //    k = 16 kb + 4 g + kk for both operands (one 16-byte LDS read each).
        const int g = lane >> 4, l16 = lane & 15;
        const float *xr = sx + (16 * w + l16) * G::LX + 4 * g;
        const float *wr = sw + l16 * G::LW + 4 * g;
        f32x4 acc[G::PT];
#pragma unroll
        for (int t = 0; t < G::PT; ++t) acc[t] = zero4();
        float sq = 0.0f;
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
            const f32x4 b = *reinterpret_cast<const f32x4 *>(xr + 16 * kb);
            sq += b[0] * b[0] + b[1] * b[1] + b[2] * b[2] + b[3] * b[3];
#pragma unroll
            for (int t = 0; t < G::PT; ++t) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(wr + t * 16 * G::LW + 16 * kb);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc[t] = mma_f32(a[kk], b[kk], acc[t]);
            }
        }
        // |x|^2 of row l16: the four lanes g of that row hold a quarter each
        sq += __shfl_xor(sq, 16, 64);
        sq += __shfl_xor(sq, 32, 64);
        float scale = 1.0f;
        if (NORM && sq > 0.0f) {
            scale = 1.0f / sqrtf(sq);
            sq = sq * scale * scale;
        }
        float *orow = so + (16 * w + l16) * G::LO;
#pragma unroll
        for (int t = 0; t < G::PT; ++t) {
            const int f0 = t * 16 + 4 * g;  // this lane's 4 projections
            if (f0 >= G::P) continue;
            f32x4 o;
            if constexpr (KIND == 1) {
                const float inv = 1.0f / sqrtf((float)F);
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = __expf(acc[t][r] * scale - 0.5f * sq) * inv;
                *reinterpret_cast<f32x4 *>(orow + f0) = o;
            } else {
                const float c = __expf(0.5f * sq) / sqrtf((float)G::P);
                f32x4 oc;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float sn, cs;
                    sincosf(acc[t][r] * scale, &sn, &cs);
                    o[r] = c * sn;
                    oc[r] = c * cs;
                }
                *reinterpret_cast<f32x4 *>(orow + f0) = o;
                *reinterpret_cast<f32x4 *>(orow + G::P + f0) = oc;
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

// ---------------------------------------------------------------------------
// Gradient of the map with respect to its input rows, dX = J(x)^T dOut row by row
// (the chain rule through the definitions above).  With y the (normalised) row:
//   elu: dy_d = dout_d * (1 for y_d > 0, exp(y_d) otherwise);
//   PRF: d out_p / dy = out_p (w_p - y), so dy = W^T a - y sum_p a_p, a_p = dout_p out_p;
//   TRF: with out_p = c sin(u_p), out_{P+p} = c cos(u_p), u_p = w_p . y, dc/dy = c y:
//        dy = W^T b + y sum_p (dout_p out_p + dout_{P+p} out_{P+p}),
//        b_p = dout_p out_{P+p} - dout_{P+p} out_p;
//   NORM: y = x / |x|, dx = (dy - y (y . dy)) / |x|; a zero row gets zero.
// One wavefront per row (lanes over the projections for u = W y, then over the
// input columns for W^T b); W is staged in LDS once per workgroup with rows of
// D + 1 floats, so that lanes reading one column of W (one row each) and lanes
// reading one row of W hit distinct banks.  Not a contraction that pays on MFMA
// at one row per wavefront; the attention backward dominates the training step.
// ---------------------------------------------------------------------------
constexpr int kFmbThreads = 256;
constexpr int kFmbWaves = kFmbThreads / 64;

__device__ __forceinline__ float fmb_wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <typename T, int D, int F, int KIND, bool NORM>
__global__ __launch_bounds__(kFmbThreads) void feature_map_backward_kernel(const T *__restrict__ X,
                                                                         const float *__restrict__ dOut,
                                                                         const float *__restrict__ W,
                                                                         float *__restrict__ dX, long rows) {
    constexpr int P = KIND == 2 ? F / 2 : F;  // projections (elu: unused)
    constexpr int LW = D + 1;
    constexpr int DL = (D + 63) / 64;  // input columns per lane
    constexpr int PL = (P + 63) / 64;  // projections per lane
    __shared__ float sW[KIND == 0 ? 1 : P * LW];
    __shared__ float sy[kFmbWaves][D];
    __shared__ float sb[kFmbWaves][KIND == 0 ? 1 : P];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if constexpr (KIND != 0) {
        for (int e = tid; e < P * D; e += kFmbThreads) sW[(e / D) * LW + e % D] = W[e];
        __syncthreads();
    }
    for (long row = (long)blockIdx.x * kFmbWaves + w; row < rows; row += (long)gridDim.x * kFmbWaves) {
        float y[DL];
        float sq = 0.0f;
#pragma unroll
        for (int j = 0; j < DL; ++j) {
            const int d = lane + 64 * j;
            y[j] = d < D ? to_f32<T>(X[row * D + d]) : 0.0f;
            sq += y[j] * y[j];
        }
        sq = fmb_wave_sum(sq);
        const float len = sqrtf(sq);
        const bool scaled = NORM && sq > 0.0f;
        if (scaled) {
            sq = 0.0f;
#pragma unroll
            for (int j = 0; j < DL; ++j) {
                y[j] /= len;
                sq += y[j] * y[j];
            }
            sq = fmb_wave_sum(sq);
        }
        const float *g = dOut + row * F;
        float dy[DL];
        if constexpr (KIND == 0) {
#pragma unroll
            for (int j = 0; j < DL; ++j) {
                const int d = lane + 64 * j;
                dy[j] = d < D ? g[d] * (y[j] > 0.0f ? 1.0f : __expf(y[j])) : 0.0f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < DL; ++j)
                if (lane + 64 * j < D) sy[w][lane + 64 * j] = y[j];
            __builtin_amdgcn_wave_barrier();
            // projections u_p = w_p . y (lanes over p), then the coefficients
            float ys = 0.0f;  // sum over the own projections of the coefficient of y
#pragma unroll
            for (int j = 0; j < PL; ++j) {
                const int pp = lane + 64 * j;
                if (pp < P) {
                    float u = 0.0f;
#pragma unroll 8
                    for (int d = 0; d < D; ++d) u += sW[pp * LW + d] * sy[w][d];
                    if constexpr (KIND == 1) {
                        const float o = __expf(u - 0.5f * sq) * (1.0f / sqrtf((float)F));
                        const float a = g[pp] * o;
                        sb[w][pp] = a;
                        ys -= a;
                    } else {
                        const float c = __expf(0.5f * sq) * (1.0f / sqrtf((float)P));
                        const float os = c * sinf(u), oc = c * cosf(u);
                        const float gs = g[pp], gc = g[P + pp];
                        sb[w][pp] = gs * oc - gc * os;
                        ys += gs * os + gc * oc;
                    }
                }
            }
            ys = fmb_wave_sum(ys);
            __builtin_amdgcn_wave_barrier();
            // dy = W^T b + y * ys (lanes over d)
#pragma unroll
            for (int j = 0; j < DL; ++j) {
                const int d = lane + 64 * j;
                float acc = 0.0f;
                if (d < D) {
#pragma unroll 8
                    for (int pp = 0; pp < P; ++pp) acc += sb[w][pp] * sW[pp * LW + d];
                }
                dy[j] = d < D ? acc + y[j] * ys : 0.0f;
            }
            __builtin_amdgcn_wave_barrier();  // sy, sb reused by this wavefront's next row
        }
        if constexpr (NORM) {
            float ydy = 0.0f;
#pragma unroll
            for (int j = 0; j < DL; ++j) ydy += y[j] * dy[j];
            ydy = fmb_wave_sum(ydy);
#pragma unroll
            for (int j = 0; j < DL; ++j) dy[j] = scaled ? (dy[j] - y[j] * ydy) / len : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < DL; ++j) {
            const int d = lane + 64 * j;
            if (d < D) dX[row * D + d] = dy[j];
        }
    }
}

template <typename T, int D, int F, int KIND>
hipError_t run_feature_map_backward(const void *X, const float *dOut, const float *W, float *dX, long rows, bool norm,
                                    hipStream_t stream) {
    if constexpr (KIND == 0 && D != F) {
        return hipErrorInvalidValue;
    } else {
        if (rows <= 0) return hipSuccess;
        const long want = (rows + kFmbWaves - 1) / kFmbWaves;
        const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
        if (norm)
            hipLaunchKernelGGL((feature_map_backward_kernel<T, D, F, KIND, true>), dim3(grid), dim3(kFmbThreads), 0,
                               stream, (const T *)X, dOut, W, dX, rows);
        else
            hipLaunchKernelGGL((feature_map_backward_kernel<T, D, F, KIND, false>), dim3(grid), dim3(kFmbThreads), 0,
                               stream, (const T *)X, dOut, W, dX, rows);
        return hipGetLastError();
    }
}

template <typename T>
hipError_t feature_map_backward_t(int D, int F, int kind, const void *X, const float *dOut, const float *W, float *dX,
                                  long rows, bool norm, hipStream_t stream) {
#define X_(D_, F_)                                                                                              \
    if (D == D_ && F == F_) {                                                                                   \
        if (kind == 1) return run_feature_map_backward<T, D_, F_, 1>(X, dOut, W, dX, rows, norm, stream);        \
        if (kind == 2) return run_feature_map_backward<T, D_, F_, 2>(X, dOut, W, dX, rows, norm, stream);        \
        if (kind == 0) return run_feature_map_backward<T, D_, F_, 0>(X, dOut, W, dX, rows, norm, stream);        \
    }
#define XF_(D_) X_(D_, 16) X_(D_, 32) X_(D_, 64) X_(D_, 128)
    XF_(16) XF_(32) XF_(64) XF_(128)
#undef XF_
#undef X_
    return hipErrorInvalidValue;
}

hipError_t feature_map_backward(int dtype, int D, int F, int kind, const void *X, const float *dOut, const float *W,
                                float *dX, long rows, bool norm, hipStream_t stream) {
    return dtype == kDtypeBf16 ? feature_map_backward_t<bf16>(D, F, kind, X, dOut, W, dX, rows, norm, stream)
                               : feature_map_backward_t<float>(D, F, kind, X, dOut, W, dX, rows, norm, stream);
}

}  // namespace la
