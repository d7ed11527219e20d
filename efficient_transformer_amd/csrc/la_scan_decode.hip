// Segment scan, zero fill, recurrent decode step, and the dtype dispatch of the
// prefill stages.
#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

// ---------------------------------------------------------------------------
// Exclusive prefix over the segment states of each head, in segment order,
// plus the total in slot G (page "Transformers are RNNs", Proposed method:
// cumulative sums).  One thread per state element; one-dimensional grid:
// block b -> head b / nblk, element block b % nblk.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void seg_scan_kernel(float *__restrict__ ws, int E, int nblk, int G, int nstates,
                                                       float *__restrict__ S_out, float *__restrict__ z_out, int DM) {
    const int bh = blockIdx.x / nblk;
    const int e = (blockIdx.x % nblk) * blockDim.x + threadIdx.x;
    if (e >= E) return;
    float *base = ws + (size_t)bh * (G + 1) * E + e;
    float run = 0.0f;
    // the loads of kScanBatch slots are issued before any of them is overwritten:
    // one memory round trip per batch instead of one per segment (same sum order)
    for (int s0 = 0; s0 < nstates; s0 += kScanBatch) {
        float x[kScanBatch];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) x[j] = s0 + j < nstates ? base[(size_t)(s0 + j) * E] : 0.0f;
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) {
            if (s0 + j < nstates) {
                base[(size_t)(s0 + j) * E] = run;
                run += x[j];
            }
        }
    }
    for (int s = nstates; s < G; ++s) base[(size_t)s * E] = run;
    base[(size_t)G * E] = run;
    if (S_out != nullptr) {
        if (e < DM)
            S_out[(size_t)bh * DM + e] = run;
        else
            z_out[(size_t)bh * (E - DM) + (e - DM)] = run;
    }
}

hipError_t prefill_scan(float *ws, int BH, int D, int M, int G, int nstates, float *S_out, float *z_out,
                        hipStream_t stream) {
    const int E = D * M + D;
    const int nblk = (E + 255) / 256;
    if (BH <= 0) return hipSuccess;
    hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)(nblk * BH)), dim3(256), 0, stream, ws, E, nblk, G, nstates,
                       S_out, z_out, D * M);
    return hipGetLastError();
}

// A fill kernel rather than hipMemsetAsync, so the call stays valid under graph capture.
__global__ __launch_bounds__(256) void fill_zero_kernel(float *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
}

hipError_t fill_zero(float *p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t prefill_fused(int dtype, int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                         void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in,
                         const float *z_in, hipStream_t stream) {
    if (dtype == (kDtypeBf16 | kOutBf16))
        return prefill_fused_bf16o(D, M, C, Q, K, V, out, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream);
    float *o32 = static_cast<float *>(out);
    return dtype == kDtypeF32    ? prefill_fused_f32(D, M, C, Q, K, V, o32, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream)
           : dtype == kDtypeBf16 ? prefill_fused_bf16(D, M, C, Q, K, V, o32, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream)
                                 : prefill_fused_feat(D, M, C, Q, K, V, o32, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream);
}

hipError_t prefill_onepass(int dtype, int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                           void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in,
                         const float *z_in, hipStream_t stream) {
    if (dtype == (kDtypeBf16 | kOutBf16))
        return prefill_onepass_bf16o(D, M, C, Q, K, V, out, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream);
    float *o32 = static_cast<float *>(out);
    return dtype == kDtypeF32    ? prefill_onepass_f32(D, M, C, Q, K, V, o32, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream)
           : dtype == kDtypeBf16 ? prefill_onepass_bf16(D, M, C, Q, K, V, o32, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream)
                                 : prefill_onepass_feat(D, M, C, Q, K, V, o32, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream);
}

bool prefill_onepass_supported(int dtype, int D, int M, int C) {
    dtype &= ~kOutBf16;  // the output type does not change the kernel's shape limits
    return dtype == kDtypeF32    ? prefill_onepass_supported_f32(D, M, C)
           : dtype == kDtypeBf16 ? prefill_onepass_supported_bf16(D, M, C)
                                 : prefill_onepass_supported_feat(D, M, C);
}

size_t prefill_lds_bytes(int dtype, int D, int M, int C) {
    dtype &= ~kOutBf16;  // the output type does not change the kernel's shape limits
    return dtype == kDtypeF32    ? prefill_lds_bytes_f32(D, M, C)
           : dtype == kDtypeBf16 ? prefill_lds_bytes_bf16(D, M, C)
                                 : prefill_lds_bytes_feat(D, M, C);
}

bool prefill_supported(int dtype, int D, int M, int C) {
    dtype &= ~kOutBf16;  // the output type does not change the kernel's shape limits
    return dtype == kDtypeF32    ? prefill_supported_f32(D, M, C)
           : dtype == kDtypeBf16 ? prefill_supported_bf16(D, M, C)
                                 : prefill_supported_feat(D, M, C);
}

hipError_t prefill_states(int dtype, int D, int M, int C, const void *K, const void *V, float *ws, int BH, int N,
                          int G, int CPS, int nstates, hipStream_t stream) {
    dtype &= ~kOutBf16;  // the states do not depend on the output type
    return dtype == kDtypeF32    ? prefill_states_f32(D, M, C, K, V, ws, BH, N, G, CPS, nstates, stream)
           : dtype == kDtypeBf16 ? prefill_states_bf16(D, M, C, K, V, ws, BH, N, G, CPS, nstates, stream)
                                 : prefill_states_feat(D, M, C, K, V, ws, BH, N, G, CPS, nstates, stream);
}

hipError_t prefill_outputs(int dtype, int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                           const float *ws, int BH, int N, int G, int CPS, int causal, float *S_out, float *z_out,
                           hipStream_t stream) {
    if (dtype == (kDtypeBf16 | kOutBf16))
        return prefill_outputs_bf16o(D, M, C, Q, K, V, out, ws, BH, N, G, CPS, causal, S_out, z_out, stream);
    float *o32 = static_cast<float *>(out);
    return dtype == kDtypeF32    ? prefill_outputs_f32(D, M, C, Q, K, V, o32, ws, BH, N, G, CPS, causal, S_out, z_out, stream)
           : dtype == kDtypeBf16 ? prefill_outputs_bf16(D, M, C, Q, K, V, o32, ws, BH, N, G, CPS, causal, S_out, z_out, stream)
                                 : prefill_outputs_feat(D, M, C, Q, K, V, o32, ws, BH, N, G, CPS, causal, S_out, z_out, stream);
}

// ---------------------------------------------------------------------------
// Recurrent decode step (page "Transformers are RNNs", Proposed method: the
// causal model is an RNN with memories S and z; Main findings: incremental
// state updates).  One workgroup per head.  Thread layout: M/4 lanes span a
// row of S with one float4 each; the workgroup covers RP rows per pass and
// PASSES passes cover all D rows, so each thread keeps D*M/(4*threads) float4
// of S in registers.  All loads of S are issued before any arithmetic, the
// state is read once and written once.
//   S += phi(k) v^T;  z += phi(k);  num = phi(q)^T S;  den = phi(q).z;  out = num/den
// ---------------------------------------------------------------------------
template <int D, int M>
struct DecCfg {
    static constexpr int NW = (D * M / 4096) > 1 ? D * M / 4096 : 1;  // wavefronts per head
    static constexpr int THREADS = 64 * NW;
    static constexpr int LPR = M / 4;                                  // lanes per row
    static constexpr int RP = THREADS / LPR;                           // rows per pass
    static constexpr int PASSES = D / RP;
    static_assert(PASSES * RP == D, "row split");
};

template <typename T>
__device__ __forceinline__ f32x4 load4(const T *p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16>(const bf16 *p) {
    bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

// DI > 0: q and k are raw rows DI wide and the random-feature map (W [P][DI],
// fkind, fnorm; as in the prefill kernels) forms their D = F features here.
template <typename T, int D, int M, bool PHI = true, int DI = 0>
__global__ __launch_bounds__((DecCfg<D, M>::THREADS)) void decode_kernel(float *__restrict__ S, float *__restrict__ z,
                                                                      const T *__restrict__ q,
                                                                      const T *__restrict__ k,
                                                                      const T *__restrict__ v,
                                                                      float *__restrict__ out,
                                                                      const float *__restrict__ W = nullptr,
                                                                      int fkind = 0, int fnorm = 0) {
    using G = DecCfg<D, M>;
    constexpr bool FEAT = DI > 0;
    constexpr int DQ = FEAT ? DI : D;  // width of the q, k rows in memory
    __shared__ float sq[D], sk[D];
    __shared__ float sx[FEAT ? 2 * DI : 1];  // raw q, k rows
    __shared__ f32x4 sred[G::NW][G::LPR];
    __shared__ float sden[G::NW];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const size_t bh = blockIdx.x;
    const int col4 = tid % G::LPR, roff = tid / G::LPR;

    f32x4 *Sh = reinterpret_cast<f32x4 *>(S + bh * D * M);
    f32x4 Sv[G::PASSES];
#pragma unroll
    for (int p = 0; p < G::PASSES; ++p) Sv[p] = __builtin_nontemporal_load(Sh + (roff + p * G::RP) * G::LPR + col4);
    const f32x4 vv = load4<T>(v + bh * M + col4 * 4);
    float zz[(D + G::THREADS - 1) / G::THREADS];
#pragma unroll
    for (int i = 0; i < (D + G::THREADS - 1) / G::THREADS; ++i) {
        const int d = tid + i * G::THREADS;
        if (d < D) {
            zz[i] = z[bh * D + d];
            if constexpr (!FEAT) {
                sq[d] = phi_if<PHI>(to_f32(q[bh * D + d]));
                sk[d] = phi_if<PHI>(to_f32(k[bh * D + d]));
            }
        }
    }
    if constexpr (FEAT) {
        for (int d = tid; d < DI; d += G::THREADS) {
            sx[d] = to_f32(q[bh * DQ + d]);
            sx[DI + d] = to_f32(k[bh * DQ + d]);
        }
        __syncthreads();
        // thread f < P: projection f of q; P <= f < 2P: of k.  Each thread also
        // sums |x|^2 of its row (LDS broadcast reads).
        const int P = fkind == 2 ? D / 2 : D;
        for (int f = tid; f < 2 * P; f += G::THREADS) {
            const int t = f / P, pf = f - t * P;
            const float *x = sx + t * DI;
            const float *wr = W + (size_t)pf * DI;
            float acc = 0.0f, ss = 0.0f;
#pragma unroll 8
            for (int d = 0; d < DI; ++d) {
                acc += wr[d] * x[d];
                ss += x[d] * x[d];
            }
            float scale = 1.0f;
            if (fnorm && ss > 0.0f) {
                scale = 1.0f / sqrtf(ss);
                ss = ss * scale * scale;
            }
            float *dst = t == 0 ? sq : sk;
            if (fkind == 1) {
                dst[pf] = __expf(acc * scale - 0.5f * ss) * (1.0f / sqrtf((float)D));
            } else {
                const float c = __expf(0.5f * ss) / sqrtf((float)P);
                float sn, cs;
                sincosf(acc * scale, &sn, &cs);
                dst[pf] = c * sn;
                dst[P + pf] = c * cs;
            }
        }
    }
    __syncthreads();

    // z += phi(k); partial den = phi(q) . z
    float den = 0.0f;
#pragma unroll
    for (int i = 0; i < (D + G::THREADS - 1) / G::THREADS; ++i) {
        const int d = tid + i * G::THREADS;
        if (d < D) {
            zz[i] += sk[d];
            z[bh * D + d] = zz[i];
            den += sq[d] * zz[i];
        }
    }

    // S += phi(k) v^T; partial num = phi(q)^T S over this thread's rows
    f32x4 num = zero4();
#pragma unroll
    for (int p = 0; p < G::PASSES; ++p) {
        const int d = roff + p * G::RP;
        const float fk = sk[d], fq = sq[d];
        f32x4 s = Sv[p];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[j] += fk * vv[j];
            num[j] += fq * s[j];
        }
        __builtin_nontemporal_store(s, Sh + d * G::LPR + col4);
    }

    // reduce num over the lanes of a wavefront that share col4, then over wavefronts
#pragma unroll
    for (int sh = G::LPR; sh < 64; sh <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) num[j] += __shfl_xor(num[j], sh, 64);
    }
    den = row_group_sum<16>(den);  // within 16-lane rows on DPP moves, then across rows
    den += __shfl_xor(den, 16, 64);
    den += __shfl_xor(den, 32, 64);
    if (G::NW > 1) {
        if (lane < G::LPR) sred[w][lane] = num;
        if (lane == 0) sden[w] = den;
        __syncthreads();
        if (w == 0 && lane < G::LPR) {
            num = sred[0][lane];
            den = sden[0];
#pragma unroll
            for (int ww = 1; ww < G::NW; ++ww) {
                const f32x4 o = sred[ww][lane];
                for (int j = 0; j < 4; ++j) num[j] += o[j];
                den += sden[ww];
            }
        }
    }
    if (w == 0 && lane < G::LPR) {
        const float inv = 1.0f / den;
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = num[j] * inv;
        *reinterpret_cast<f32x4 *>(out + bh * M + lane * 4) = o;
    }
}

template <typename T, int D, int M, bool PHI = true>
hipError_t run_decode(float *S, float *z, const void *q, const void *k, const void *v, float *out, int BH,
                      hipStream_t stream) {
    if (BH <= 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<T, D, M, PHI>), dim3((unsigned)BH), dim3(DecCfg<D, M>::THREADS), 0, stream, S, z,
                       (const T *)q, (const T *)k, (const T *)v, out, nullptr, 0, 0);
    return hipGetLastError();
}

template <typename T, int DI, int F, int M>
hipError_t run_decode_features(float *S, float *z, const void *q, const void *k, const void *v, float *out,
                               const float *W, int kind, int norm, int BH, hipStream_t stream) {
    if (BH <= 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<T, F, M, false, DI>), dim3((unsigned)BH), dim3(DecCfg<F, M>::THREADS), 0, stream,
                       S, z, (const T *)q, (const T *)k, (const T *)v, out, W, kind, norm);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Recurrent decode over T consecutive tokens of every head, the state held in
// registers for the whole call (read once, written once).  The same RNN step as
// decode_kernel, repeated: for t = 0..T-1
//   S += phi(k_t) v_t^T;  z += phi(k_t);  out_t = phi(q_t)^T S / phi(q_t).z
// Thread layout as decode_kernel; each thread also keeps z of its own rows (the
// rows d = roff + p*RP, replicated over the LPR lanes of a row), so phi(q).z is
// reduced together with the numerator.  Tokens are staged TB at a time in LDS
// (phi applied once); q, k [BH][T][D], v, out [BH][T][M].
// ---------------------------------------------------------------------------
constexpr int kDecodeTokenBlock = 16;

template <typename T, int D, int M, bool PHI = true>
__global__ __launch_bounds__((DecCfg<D, M>::THREADS)) void decode_steps_kernel(
    float *__restrict__ S, float *__restrict__ z, const T *__restrict__ q, const T *__restrict__ k,
    const T *__restrict__ v, float *__restrict__ out, int Tn) {
    using G = DecCfg<D, M>;
    constexpr int TB = kDecodeTokenBlock;
    __shared__ float sq[TB][D], sk[TB][D];
    __shared__ f32x4 sv[TB][G::LPR];
    __shared__ f32x4 sred[2][G::NW][G::LPR];
    __shared__ float sden[2][G::NW];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const size_t bh = blockIdx.x;
    const int col4 = tid % G::LPR, roff = tid / G::LPR;

    f32x4 *Sh = reinterpret_cast<f32x4 *>(S + bh * D * M);
    f32x4 Sv[G::PASSES];
    float zl[G::PASSES];
#pragma unroll
    for (int p = 0; p < G::PASSES; ++p) {
        Sv[p] = __builtin_nontemporal_load(Sh + (roff + p * G::RP) * G::LPR + col4);
        zl[p] = z[bh * D + roff + p * G::RP];
    }
    const size_t tok0 = bh * (size_t)Tn;
    for (int t0 = 0; t0 < Tn; t0 += TB) {
        const int nt = min(TB, Tn - t0);
        __syncthreads();  // the previous block's readers are done
        const T *qb = q + (tok0 + t0) * D, *kb = k + (tok0 + t0) * D;
        for (int e = tid; e < nt * D; e += G::THREADS) {
            sq[e / D][e % D] = phi_if<PHI>(to_f32(qb[e]));
            sk[e / D][e % D] = phi_if<PHI>(to_f32(kb[e]));
        }
        const T *vb = v + (tok0 + t0) * M;
        for (int e = tid; e < nt * G::LPR; e += G::THREADS) sv[e / G::LPR][e % G::LPR] = load4<T>(vb + e * 4);
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            const f32x4 vv = sv[t][col4];
            f32x4 num = zero4();
            float dn = 0.0f;
#pragma unroll
            for (int p = 0; p < G::PASSES; ++p) {
                const int d = roff + p * G::RP;
                const float fk = sk[t][d], fq = sq[t][d];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    Sv[p][j] += fk * vv[j];
                    num[j] += fq * Sv[p][j];
                }
                zl[p] += fk;
                dn += fq * zl[p];
            }
            // sum over the lanes of the wavefront that share col4 (distinct rows)
#pragma unroll
            for (int sh = G::LPR; sh < 64; sh <<= 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) num[j] += __shfl_xor(num[j], sh, 64);
                dn += __shfl_xor(dn, sh, 64);
            }
            if (G::NW > 1) {
                const int buf = t & 1;  // two buffers: one barrier per token
                if (lane < G::LPR) sred[buf][w][lane] = num;
                if (lane == 0) sden[buf][w] = dn;
                __syncthreads();
                if (w == 0 && lane < G::LPR) {
                    num = sred[buf][0][lane];
                    dn = sden[buf][0];
#pragma unroll
                    for (int ww = 1; ww < G::NW; ++ww) {
                        const f32x4 o = sred[buf][ww][lane];
#pragma unroll
                        for (int j = 0; j < 4; ++j) num[j] += o[j];
                        dn += sden[buf][ww];
                    }
                }
            }
            if (w == 0 && lane < G::LPR) {
                const float inv = 1.0f / dn;
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = num[j] * inv;
                *reinterpret_cast<f32x4 *>(out + (tok0 + t0 + t) * M + lane * 4) = o;
            }
        }
    }
#pragma unroll
    for (int p = 0; p < G::PASSES; ++p) {
        __builtin_nontemporal_store(Sv[p], Sh + (roff + p * G::RP) * G::LPR + col4);
        if (col4 == 0) z[bh * D + roff + p * G::RP] = zl[p];
    }
}

template <typename T, int D, int M, bool PHI = true>
hipError_t run_decode_steps(float *S, float *z, const void *q, const void *k, const void *v, float *out, int BH,
                            int Tn, hipStream_t stream) {
    if (BH <= 0 || Tn <= 0) return hipSuccess;
    hipLaunchKernelGGL((decode_steps_kernel<T, D, M, PHI>), dim3((unsigned)BH), dim3(DecCfg<D, M>::THREADS), 0, stream,
                       S, z, (const T *)q, (const T *)k, (const T *)v, out, Tn);
    return hipGetLastError();
}

hipError_t decode_steps(int dtype, int D, int M, float *S, float *z, const void *q, const void *k, const void *v,
                        float *out, int BH, int Tn, hipStream_t stream) {
#define X(D_, M_)                                                                                  \
    if (D == D_ && M == M_)                                                                        \
        return dtype == kDtypeF32   ? run_decode_steps<float, D_, M_>(S, z, q, k, v, out, BH, Tn, stream) \
               : dtype == kDtypeBf16 ? run_decode_steps<bf16, D_, M_>(S, z, q, k, v, out, BH, Tn, stream)  \
                                     : run_decode_steps<float, D_, M_, false>(S, z, q, k, v, out, BH, Tn, stream);
#define XM(D_) X(D_, 16) X(D_, 32) X(D_, 64) X(D_, 128)
    XM(16) XM(32) XM(64) XM(128)
#undef XM
#undef X
    return hipErrorInvalidValue;
}

hipError_t decode_step(int dtype, int D, int M, float *S, float *z, const void *q, const void *k, const void *v,
                       float *out, int BH, hipStream_t stream) {
#define X(D_, M_)                                                                        \
    if (D == D_ && M == M_)                                                              \
        return dtype == kDtypeF32   ? run_decode<float, D_, M_>(S, z, q, k, v, out, BH, stream) \
               : dtype == kDtypeBf16 ? run_decode<bf16, D_, M_>(S, z, q, k, v, out, BH, stream)  \
                                     : run_decode<float, D_, M_, false>(S, z, q, k, v, out, BH, stream);
#define XM(D_) X(D_, 16) X(D_, 32) X(D_, 64) X(D_, 128)
    XM(16) XM(32) XM(64) XM(128)
#undef XM
#undef X
    return hipErrorInvalidValue;
}

hipError_t decode_step_features(int dtype, int DI, int F, int M, float *S, float *z, const void *q, const void *k,
                                const void *v, float *out, const float *W, int kind, int norm, int BH,
                                hipStream_t stream) {
#define X(DI_, F_, M_)                                                                                        \
    if (DI == DI_ && F == F_ && M == M_)                                                                      \
        return dtype == kDtypeF32                                                                             \
                   ? run_decode_features<float, DI_, F_, M_>(S, z, q, k, v, out, W, kind, norm, BH, stream)  \
                   : run_decode_features<bf16, DI_, F_, M_>(S, z, q, k, v, out, W, kind, norm, BH, stream);
#define XM(DI_, F_) X(DI_, F_, 16) X(DI_, F_, 32) X(DI_, F_, 64) X(DI_, F_, 128)
#define XF(DI_) XM(DI_, 16) XM(DI_, 32) XM(DI_, 64)
    XF(16) XF(32) XF(64) XF(128)
#undef XF
#undef XM
#undef X
    return hipErrorInvalidValue;
}

}  // namespace la
