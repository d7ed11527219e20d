// Device-side building blocks for the linear-attention kernels (gfx950 / CDNA4).
//
// MFMA operand layouts used throughout (64-lane wavefront, lane = 16*g + l16):
//   v_mfma_f32_16x16x4_f32     A: lane holds A[l16][g]          B: B[g][l16]
//   v_mfma_f32_16x16x32_bf16   A: lane holds A[l16][8g .. 8g+7] B: B[8g .. 8g+7][l16]
//   result (both)              lane holds C[4g + r][l16], r = 0..3
// The contraction index may be permuted freely as long as A and B use the same
// permutation, which the tile routines exploit to avoid register transposes.
//
// Only one MFMA shape per element type is used.  A 16-deep bf16 contraction is
// done as a 32-deep one with the upper half of every lane's slots zero: chaining
// v_mfma_f32_16x16x16_bf16 and v_mfma_f32_16x16x32_bf16 on one accumulator, with
// no wait states between them in the generated code, gave wrong values in half
// of the result rows on gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy bits of buffer stores: sc1 = agent scope (write-through past the
// per-XCD L2, so another XCD reads the stored value from memory).
constexpr int kCachePolicyAgent = 16;
// Segment states read per memory round trip by the element-wise state scans.
constexpr int kScanBatch = 8;
using bf16 = __bf16;

// phi(x) = elu(x) + 1: x + 1 for x > 0, exp(x) otherwise (page "Transformers are
// RNNs", Main findings: elu-based feature map).  Written as max(x + 1, exp(-|x|)):
// for x > 0, exp(-x) < 1 < x + 1; for x <= 0, exp(x) >= 1 + x, and -|x| = x.  Four
// VALU operations (the negated absolute value is a source modifier of the scaling
// multiply) instead of a compare and a select on top of the same three; -inf
// maps to exactly 0.
__device__ __forceinline__ float phi(float x) { return fmaxf(x + 1.0f, __expf(-fabsf(x))); }
// phi when P, else the identity (the input already holds features).
template <bool P>
__device__ __forceinline__ float phi_if(float x) {
    if constexpr (P) return phi(x);
    else return x;
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// value after a round trip through T (identity for float)
template <typename T> __device__ __forceinline__ float round_as(float x) { return to_f32<T>(from_f32<T>(x)); }

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// a 16-deep contraction on the 32-deep instruction: slots 4..7 of every lane are zero
__device__ __forceinline__ f32x4 mma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16 zero = (bf16)0.0f;
    bf16x8 a8 = {a[0], a[1], a[2], a[3], zero, zero, zero, zero};
    bf16x8 b8 = {b[0], b[1], b[2], b[3], zero, zero, zero, zero};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// fp32 variant with strided operands: for contraction index k = 4*ks + g the lane
// reads A at a[k * a_ks] (a points at row l16 of A) and B at b[k * b_ks] (b points
// at column l16 of B).
template <int K>
__device__ __forceinline__ f32x4 tile_dot_f32(const float *a, int a_ks, const float *b, int b_ks, int g,
                                              f32x4 acc) {
    static_assert(K % 4 == 0, "K must be a multiple of 4");
#pragma unroll
    for (int ks = 0; ks < K / 4; ++ks) {
        const int k = 4 * ks + g;
        acc = mma_f32(a[k * a_ks], b[k * b_ks], acc);
    }
    return acc;
}

// x of another lane of the same 16-lane row, by a DPP move (a VALU operation; no LDS
// traffic): CTRL 0xB1 / 0x4E swap lanes i and i^1 / i^2 within each quad, 0x141 mirrors
// each half-row (lane i of 8 reads lane 7 - i), 0x140 mirrors the row (i reads 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// sum of x over each aligned group of N consecutive lanes (N = 1, 2, 4, 8 or 16), in
// every lane of the group: the quad sums by two swaps, then the half-row mirror adds
// the other quad's sum and the row mirror the other half-row's
template <int N>
__device__ __forceinline__ float row_group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1, 2, 4, 8 or 16 lanes");
    if constexpr (N >= 2) x += dpp_move<0xB1>(x);
    if constexpr (N >= 4) x += dpp_move<0x4E>(x);
    if constexpr (N >= 8) x += dpp_move<0x141>(x);
    if constexpr (N >= 16) x += dpp_move<0x140>(x);
    return x;
}

// Shifts for scans over lanes, by DPP moves; lanes without a source lane get `fill`:
// row_shr (0x110 + O): lane i reads lane i - O of its own 16-lane row;
// row_bcast:15 (0x142, written in rows 1 and 3 only): every lane of a row reads lane
// 15 of the row before; wave_shr:1 (0x138): lane i reads lane i - 1 of the wavefront.
template <int O>
__device__ __forceinline__ float dpp_row_shr(float x, float fill) {
    static_assert(O >= 1 && O <= 15, "shift within a row");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, x),
                                                                 0x110 + O, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_row_bcast15(float x, float fill) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, x),
                                                                 0x142, 0xA, 0xF, false));
}
__device__ __forceinline__ float dpp_wave_shr1(float x, float fill) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, x),
                                                                 0x138, 0xF, 0xF, false));
}

// sum of x over the four lanes {l16, l16+16, l16+32, l16+48}
__device__ __forceinline__ float sum_over_groups(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

}  // namespace la
