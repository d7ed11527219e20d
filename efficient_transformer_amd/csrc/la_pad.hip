// Widths without a specialised kernel: D or M a multiple of 16 below 128 that is
// not a power of two (48, 80, 96, 112).
//
// Prefill: the rows are copied into tiles of the next supported width (64 or
// 128) and the specialised kernels run on those.  The extra feature columns
// of Q and K are filled with -inf, so that phi = elu + 1 maps them to exactly
// zero (phi(x) = exp(x) for x <= 0, and exp(-inf) = 0): they add nothing to
// phi(q) . phi(k), to S or to z (page "Transformers are RNNs", Proposed method:
// the similarity is the dot product of the feature vectors, so zero features
// drop out).  The extra value columns are zero; their outputs are never copied
// back.  Inputs that already hold features (no map) are padded with zeros.
//
// Decode: one generic kernel with the widths as arguments (decode_any_kernel).
#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

namespace {

constexpr int kPadThreads = 256;

// dst[h][r][c] = src[h][r][c] for r < Rs and c < Cs, else `fill` in every
// 32-bit word; rows of Cs (source) and Cd (destination) 16-byte units.
__global__ __launch_bounds__(kPadThreads) void pad_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                          long BH, long Rs, long Cs, long Rd, long Cd,
                                                          unsigned fill) {
    const long total = BH * Rd * Cd;
    const long step = (long)gridDim.x * kPadThreads;
    for (long i = (long)blockIdx.x * kPadThreads + threadIdx.x; i < total; i += step) {
        const long c = i % Cd, rr = i / Cd;
        const long r = rr % Rd, h = rr / Rd;
        u32x4 v = {fill, fill, fill, fill};
        if (r < Rs && c < Cs) v = __builtin_nontemporal_load(src + (h * Rs + r) * Cs + c);
        dst[i] = v;
    }
}

// dst[h][r][c] = src[h][r][c] for r < Rs, c < Cs (src rows Cd units, Rd rows per h)
__global__ __launch_bounds__(kPadThreads) void unpad_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                            long BH, long Rs, long Cs, long Rd, long Cd) {
    const long total = BH * Rs * Cs;
    const long step = (long)gridDim.x * kPadThreads;
    for (long i = (long)blockIdx.x * kPadThreads + threadIdx.x; i < total; i += step) {
        const long c = i % Cs, rr = i / Cs;
        const long r = rr % Rs, h = rr / Rs;
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + (h * Rd + r) * Cd + c), dst + i);
    }
}

// dst[i] = src[i] widened from bf16 to fp32, eight values per item
__global__ __launch_bounds__(kPadThreads) void widen_kernel(const u32x4 *__restrict__ src, f32x4 *__restrict__ dst,
                                                            long items) {
    const long step = (long)gridDim.x * kPadThreads;
    for (long i = (long)blockIdx.x * kPadThreads + threadIdx.x; i < items; i += step) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        f32x4 lo, hi;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            lo[2 * j] = __builtin_bit_cast(float, v[j] << 16);
            lo[2 * j + 1] = __builtin_bit_cast(float, v[j] & 0xffff0000u);
            hi[2 * j] = __builtin_bit_cast(float, v[2 + j] << 16);
            hi[2 * j + 1] = __builtin_bit_cast(float, v[2 + j] & 0xffff0000u);
        }
        __builtin_nontemporal_store(lo, dst + 2 * i);
        __builtin_nontemporal_store(hi, dst + 2 * i + 1);
    }
}

unsigned grid_for(long units) {
    const long b = (units + kPadThreads - 1) / kPadThreads;
    return (unsigned)(b < 256 * 16 ? (b > 0 ? b : 1) : 256 * 16);
}

template <typename T>
__device__ __forceinline__ f32x4 load4_any(const T *p);
template <>
__device__ __forceinline__ f32x4 load4_any<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <>
__device__ __forceinline__ f32x4 load4_any<bf16>(const bf16 *p) {
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

// Recurrent steps of Tn tokens of every head (page "Transformers are RNNs",
// Proposed method: the causal model is an RNN with memories S and z):
//   S += phi(k) v^T;  z += phi(k);  out = phi(q)^T S / phi(q) . z
// D, M: multiples of 16 up to 128, given at run time.  One workgroup of 256
// threads per head.  Thread (roff, col4) keeps the float4 column group col4 of
// rows roff, roff + RP, ... of S in registers for the whole call (RP = 256 / (M/4)
// rows per pass, at least 8, so at most 16 passes); thread d < D keeps z[d].
// Per token the partial numerators meet in LDS and are summed in row order;
// the denominator phi(q) . z is summed in order over d.  q, k: [BH][Tn][D];
// v, out: [BH][Tn][M].  The state is read once and written once per call, with
// nontemporal accesses.
constexpr int kAnyMaxPasses = 16;

template <typename T, bool PHI>
__global__ __launch_bounds__(kPadThreads) void decode_any_kernel(float *__restrict__ S, float *__restrict__ z,
                                                                 const T *__restrict__ q, const T *__restrict__ k,
                                                                 const T *__restrict__ v, float *__restrict__ out,
                                                                 int D, int M, int Tn) {
    __shared__ float sq[128], sk[128], sz[128];
    __shared__ f32x4 sred[kPadThreads];
    const int tid = threadIdx.x;
    const size_t bh = blockIdx.x;
    const int LPR = M / 4;
    const int RP = kPadThreads / LPR;
    const int col4 = tid % LPR, roff = tid / LPR;
    const bool active = roff < RP;
    f32x4 *Sh = reinterpret_cast<f32x4 *>(S + bh * (size_t)D * M);
    f32x4 Sv[kAnyMaxPasses];
#pragma unroll
    for (int p = 0; p < kAnyMaxPasses; ++p) {
        const int d = roff + p * RP;
        Sv[p] = (active && d < D) ? __builtin_nontemporal_load(Sh + (size_t)d * LPR + col4) : zero4();
    }
    float zz = tid < D ? z[bh * D + tid] : 0.0f;
    for (int t = 0; t < Tn; ++t) {
        const size_t tok = bh * (size_t)Tn + t;
        if (tid < D) {
            const float fk = phi_if<PHI>(to_f32(k[tok * D + tid]));
            sq[tid] = phi_if<PHI>(to_f32(q[tok * D + tid]));
            sk[tid] = fk;
            zz += fk;
            sz[tid] = zz;
        }
        const f32x4 vv = active ? load4_any<T>(v + tok * M + col4 * 4) : zero4();
        __syncthreads();
        f32x4 num = zero4();
#pragma unroll
        for (int p = 0; p < kAnyMaxPasses; ++p) {
            const int d = roff + p * RP;
            if (active && d < D) {
                const float fk = sk[d], fq = sq[d];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    Sv[p][j] += fk * vv[j];
                    num[j] += fq * Sv[p][j];
                }
            }
        }
        sred[tid] = num;
        __syncthreads();
        if (tid < LPR) {
            f32x4 acc = zero4();
            for (int r = 0; r < RP; ++r) acc += sred[r * LPR + tid];
            float den = 0.0f;
            for (int d = 0; d < D; ++d) den += sq[d] * sz[d];
            const float inv = 1.0f / den;
            *reinterpret_cast<f32x4 *>(out + tok * M + tid * 4) = acc * inv;
        }
        __syncthreads();  // LDS is rewritten by the next token
    }
#pragma unroll
    for (int p = 0; p < kAnyMaxPasses; ++p) {
        const int d = roff + p * RP;
        if (active && d < D) __builtin_nontemporal_store(Sv[p], Sh + (size_t)d * LPR + col4);
    }
    if (tid < D) z[bh * D + tid] = zz;
}

}  // namespace

hipError_t pad_copy(const void *src, void *dst, long BH, long Rs, long Cs_bytes, long Rd, long Cd_bytes,
                    unsigned fill, hipStream_t stream) {
    const long Cs = Cs_bytes / 16, Cd = Cd_bytes / 16;
    const long units = BH * Rd * Cd;
    if (units <= 0) return hipSuccess;
    hipLaunchKernelGGL(pad_kernel, dim3(grid_for(units)), dim3(kPadThreads), 0, stream,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), BH, Rs, Cs, Rd, Cd, fill);
    return hipGetLastError();
}

hipError_t unpad_copy(const void *src, void *dst, long BH, long Rs, long Cs_bytes, long Rd, long Cd_bytes,
                      hipStream_t stream) {
    const long Cs = Cs_bytes / 16, Cd = Cd_bytes / 16;
    const long units = BH * Rs * Cs;
    if (units <= 0) return hipSuccess;
    hipLaunchKernelGGL(unpad_kernel, dim3(grid_for(units)), dim3(kPadThreads), 0, stream,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), BH, Rs, Cs, Rd, Cd);
    return hipGetLastError();
}

hipError_t widen_bf16(const void *src, float *dst, long n, hipStream_t stream) {
    if (n % 8) return hipErrorInvalidValue;
    const long items = n / 8;
    if (items <= 0) return hipSuccess;
    hipLaunchKernelGGL(widen_kernel, dim3(grid_for(items)), dim3(kPadThreads), 0, stream,
                       static_cast<const u32x4 *>(src), reinterpret_cast<f32x4 *>(dst), items);
    return hipGetLastError();
}

hipError_t decode_any(int dtype, int D, int M, float *S, float *z, const void *q, const void *k, const void *v,
                      float *out, int BH, int Tn, hipStream_t stream) {
    if (BH <= 0 || Tn <= 0) return hipSuccess;
    if (D % 16 || M % 16 || D < 16 || M < 16 || D > 128 || M > 128) return hipErrorInvalidValue;
    if (dtype == kDtypeBf16)
        hipLaunchKernelGGL((decode_any_kernel<bf16, true>), dim3((unsigned)BH), dim3(kPadThreads), 0, stream, S, z,
                           static_cast<const bf16 *>(q), static_cast<const bf16 *>(k), static_cast<const bf16 *>(v),
                           out, D, M, Tn);
    else if (dtype == kDtypeF32)
        hipLaunchKernelGGL((decode_any_kernel<float, true>), dim3((unsigned)BH), dim3(kPadThreads), 0, stream, S, z,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), out, D, M, Tn);
    else
        hipLaunchKernelGGL((decode_any_kernel<float, false>), dim3((unsigned)BH), dim3(kPadThreads), 0, stream, S, z,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), out, D, M, Tn);
    return hipGetLastError();
}

}  // namespace la
