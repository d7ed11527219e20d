// Parallel (prefill) mode of causal kernelized linear attention.
//
// Page "Transformers are RNNs" (Katharopoulos et al., 2020), Proposed method:
// attention with the similarity phi(q)^T phi(k) is rewritten by associativity as
// phi(Q) (phi(K)^T V); causal masking is kept by the cumulative sums S_i, Z_i.
// Here each head's sequence is cut into chunks of C positions and the chunks
// into segments.  Within a chunk the masked quadratic term is formed on MFMA;
// across chunks the state (S, z) carries the sums; across segments an exclusive
// prefix of per-segment states links the pieces.  Per chunk c with state
// (S, z) of all earlier positions:
//   A   = tril(phi(Q_c) phi(K_c)^T)               (C x C, diagonal kept)
//   num = A V_c + phi(Q_c) S                      (C x M)
//   den = rowsum(A) + phi(Q_c) z                  (C)
//   out = num / den
//   S  += phi(K_c)^T V_c ;  z += colsum(phi(K_c))
//
// One workgroup (4 wavefronts) walks one segment chunk by chunk, keeping S in
// MFMA accumulators and a copy in LDS for the read-out of the next chunk.
//
// LDS layouts (element type T):
//   fp32 : phi(Q) [C][D+4], phi(K) [C][D+4], V [C][M+4], S [D][M+4]
//   bf16 : phi(Q) [C][D+8], phi(K) [C][D+8], phi(K)^T [D][C+8], V^T [M][C+8],
//          S^T [M][D+8]
//   z (fp32, rounded like S) [D]
// bf16 MFMA operands need the contraction index contiguous per lane, hence the
// transposed copies; fp32 MFMA takes one element per lane and reads the
// natural layouts with strides.
#pragma once

#include <type_traits>

#include "la_device.hpp"

namespace la {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr size_t kMaxLds = 160 * 1024;

template <typename T, int D, int M, int C>
struct Cfg {
    static constexpr bool F32 = std::is_same<T, float>::value;
    static constexpr int RT = C / 16, DT = D / 16, MT = M / 16;
    static constexpr int NWR = RT < kWaves ? RT : kWaves;  // wave groups over row tiles
    static constexpr int NWM = kWaves / NWR;               // wave groups over m tiles
    static constexpr int S_TILES = DT * MT;
    static constexpr int S_PER_WAVE = (S_TILES + kWaves - 1) / kWaves;
    static constexpr int PAD = F32 ? 4 : 8;
    static constexpr int LQ = D + PAD;  // row stride of phi(Q), phi(K) (and S^T for bf16)
    static constexpr int LV = M + PAD;  // fp32: row stride of V and S
    static constexpr int LT = C + PAD;  // bf16: row stride of phi(K)^T and V^T
    static constexpr int E = D * M + D;  // floats per state slot

    // element offsets of the output kernel's LDS carve-up
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + C * LQ;
    static constexpr int oV = oK + C * LQ;                 // fp32: V; bf16: V^T
    static constexpr int nV = F32 ? C * LV : M * LT;
    static constexpr int oKt = oV + nV;                    // bf16 only
    static constexpr int nKt = F32 ? 0 : D * LT;
    static constexpr int oS = oKt + nKt;                   // fp32: S; bf16: S^T
    static constexpr int nS = F32 ? D * LV : M * LQ;
    static constexpr int nT_out = oS + nS;
    static constexpr size_t out_bytes = ((nT_out * sizeof(T) + 15) / 16) * 16 + D * sizeof(float);

    // state kernel: fp32 phi(K) [C][LQ] + V [C][LV]; bf16 phi(K)^T [D][LT] + V^T [M][LT]
    static constexpr int sK_n = F32 ? C * LQ : D * LT;
    static constexpr int sV_n = F32 ? C * LV : M * LT;
    static constexpr size_t state_bytes = (sK_n + sV_n) * sizeof(T);

    static constexpr bool fits = out_bytes <= kMaxLds && state_bytes <= kMaxLds;
};

// ---------------------------------------------------------------------------
// Staging of a C x W tile of a [N][W] head matrix: global -> registers -> LDS.
// fp32: an item is one 16-byte vector of one row (rows of W/4 items).
// bf16: an item is one 16-byte column block of four consecutive rows, so that
//       the transposed store can write four keys of one column at once.
// Rows at or beyond N are stored as zeros (after phi, so they add nothing).
// ---------------------------------------------------------------------------
template <typename T, int C, int W>
struct Stage {
    static constexpr bool F32 = std::is_same<T, float>::value;
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr int NV = W / VEC;
    static constexpr int RPI = F32 ? 1 : 4;
    static constexpr int ITEMS = (C / RPI) * NV;
    static constexpr int PER = (ITEMS + kThreads - 1) / kThreads;
    uint4 r[PER][RPI];

    __device__ __forceinline__ void load(const T *__restrict__ head, int row0, int N, int tid) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int item = tid + p * kThreads;
            if (ITEMS % kThreads == 0 || item < ITEMS) {
                const int rq = item / NV, cv = item % NV;
#pragma unroll
                for (int i = 0; i < RPI; ++i) {
                    const int grow = row0 + rq * RPI + i;
                    r[p][i] = grow < N ? *reinterpret_cast<const uint4 *>(head + (size_t)grow * W + cv * VEC)
                                       : make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }
    }

    // natural layout dst[row][col], optionally through phi
    template <bool PHI>
    __device__ __forceinline__ void store_natural(T *dst, int ld, int row0, int N, int tid) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int item = tid + p * kThreads;
            if (ITEMS % kThreads == 0 || item < ITEMS) {
                const int rq = item / NV, cv = item % NV;
#pragma unroll
                for (int i = 0; i < RPI; ++i) {
                    const int row = rq * RPI + i;
                    const bool ok = row0 + row < N;
                    if constexpr (F32) {
                        f32x4 x = __builtin_bit_cast(f32x4, r[p][i]);
                        f32x4 y;
#pragma unroll
                        for (int j = 0; j < 4; ++j) y[j] = ok ? (PHI ? phi(x[j]) : x[j]) : 0.0f;
                        *reinterpret_cast<f32x4 *>(dst + row * ld + cv * 4) = y;
                    } else {
                        bf16x8 x = __builtin_bit_cast(bf16x8, r[p][i]);
                        bf16x8 y;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float f = (float)x[j];
                            y[j] = (bf16)(ok ? (PHI ? phi(f) : f) : 0.0f);
                        }
                        *reinterpret_cast<bf16x8 *>(dst + row * ld + cv * 8) = y;
                    }
                }
            }
        }
    }

    // bf16 only: transposed layout dst[col][row] (and optionally the natural one too)
    template <bool PHI, bool ALSO_NATURAL>
    __device__ __forceinline__ void store_transposed(T *dst_t, int ldt, T *dst_n, int ldn, int row0, int N,
                                                     int tid) const {
        static_assert(!F32, "transposed staging is for bf16 operands");
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int item = tid + p * kThreads;
            if (ITEMS % kThreads == 0 || item < ITEMS) {
                const int rq = item / NV, cv = item % NV;
                bf16x8 y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = row0 + rq * 4 + i < N;
                    bf16x8 x = __builtin_bit_cast(bf16x8, r[p][i]);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float f = (float)x[j];
                        y[i][j] = (bf16)(ok ? (PHI ? phi(f) : f) : 0.0f);
                    }
                    if constexpr (ALSO_NATURAL)
                        *reinterpret_cast<bf16x8 *>(dst_n + (rq * 4 + i) * ldn + cv * 8) = y[i];
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    bf16x4 t = {y[0][j], y[1][j], y[2][j], y[3][j]};
                    *reinterpret_cast<bf16x4 *>(dst_t + (cv * 8 + j) * ldt + rq * 4) = t;
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// State update S += phi(K_c)^T V_c for the S tiles this wavefront owns
// (tile t = w + kWaves*i, t = dt*MT + mt); result lane layout
// acc[i][r] = S[dt*16 + 4g + r][mt*16 + l16].
// ---------------------------------------------------------------------------
template <typename T, int D, int M, int C, int NS>
__device__ __forceinline__ void state_update(f32x4 (&acc)[NS], const T *sKx,
                                             const T *sVx, int w, int g, int l16) {
    using G = Cfg<T, D, M, C>;
#pragma unroll
    for (int i = 0; i < G::S_PER_WAVE; ++i) {
        const int t = w + kWaves * i;
        if (G::S_TILES % kWaves == 0 || t < G::S_TILES) {
            const int dt = t / G::MT, mt = t % G::MT;
            if constexpr (G::F32) {
                // A = phi(K)^T: row d, contraction over keys -> sK[key][d]
                acc[i] = tile_dot_f32<C>(sKx + dt * 16 + l16, G::LQ, sVx + mt * 16 + l16, G::LV, g, acc[i]);
            } else {
                acc[i] = tile_dot_bf16<C>(sKx + (dt * 16 + l16) * G::LT, sVx + (mt * 16 + l16) * G::LT, g, acc[i]);
            }
        }
    }
}

// column sums of phi(K_c) for z (thread tid < D owns z[tid])
template <typename T, int D, int M, int C>
__device__ __forceinline__ float z_update(float z, const T *sKx, int tid) {
    using G = Cfg<T, D, M, C>;
    if (tid < D) {
#pragma unroll 8
        for (int key = 0; key < C; ++key) {
            if constexpr (G::F32)
                z += sKx[key * G::LQ + tid];
            else
                z += to_f32(sKx[tid * G::LT + key]);
        }
    }
    return z;
}

// Copy the register state into the LDS read-out copy (rounded to T).
template <typename T, int D, int M, int C, int NS>
__device__ __forceinline__ void state_to_lds(const f32x4 (&acc)[NS], float z, T *sS,
                                             float *sz, int w, int g, int l16, int tid) {
    using G = Cfg<T, D, M, C>;
#pragma unroll
    for (int i = 0; i < G::S_PER_WAVE; ++i) {
        const int t = w + kWaves * i;
        if (G::S_TILES % kWaves == 0 || t < G::S_TILES) {
            const int dt = t / G::MT, mt = t % G::MT;
            if constexpr (G::F32) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[(dt * 16 + 4 * g + r) * G::LV + mt * 16 + l16] = acc[i][r];
            } else {
                bf16x4 v = {(bf16)acc[i][0], (bf16)acc[i][1], (bf16)acc[i][2], (bf16)acc[i][3]};
                *reinterpret_cast<bf16x4 *>(sS + (mt * 16 + l16) * G::LQ + dt * 16 + 4 * g) = v;
            }
        }
    }
    if (tid < D) sz[tid] = round_as<T>(z);
}

// Load a state slot ([D][M] then [D], fp32) into the register layout.
template <typename T, int D, int M, int C, int NS>
__device__ __forceinline__ void state_from_global(f32x4 (&acc)[NS], float &z,
                                                  const float *st, int w, int g, int l16, int tid) {
    using G = Cfg<T, D, M, C>;
#pragma unroll
    for (int i = 0; i < G::S_PER_WAVE; ++i) {
        const int t = w + kWaves * i;
        acc[i] = zero4();
        if (G::S_TILES % kWaves == 0 || t < G::S_TILES) {
            const int dt = t / G::MT, mt = t % G::MT;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] = st[(dt * 16 + 4 * g + r) * M + mt * 16 + l16];
        }
    }
    z = tid < D ? st[D * M + tid] : 0.0f;
}

template <typename T, int D, int M, int C, int NS>
__device__ __forceinline__ void state_to_global(const f32x4 (&acc)[NS], float z,
                                                float *S, float *zp, int w, int g, int l16, int tid) {
    using G = Cfg<T, D, M, C>;
#pragma unroll
    for (int i = 0; i < G::S_PER_WAVE; ++i) {
        const int t = w + kWaves * i;
        if (G::S_TILES % kWaves == 0 || t < G::S_TILES) {
            const int dt = t / G::MT, mt = t % G::MT;
#pragma unroll
            for (int r = 0; r < 4; ++r) S[(dt * 16 + 4 * g + r) * M + mt * 16 + l16] = acc[i][r];
        }
    }
    if (tid < D) zp[tid] = z;
}

// ---------------------------------------------------------------------------
// Stage 1: per-segment summed state (S, z) of phi(k_j) v_j^T, phi(k_j).
// Grid: BH * nstates workgroups; workgroup -> (bh, s).
// ---------------------------------------------------------------------------
template <typename T, int D, int M, int C>
__global__ __launch_bounds__(kThreads) void seg_state_kernel(const T *__restrict__ K, const T *__restrict__ V,
                                                             float *__restrict__ ws, int N, int G_, int CPS,
                                                             int nstates) {
    using G = Cfg<T, D, M, C>;
    __shared__ __attribute__((aligned(16))) T smem[G::sK_n + G::sV_n];
    T *sKx = smem;
    T *sVx = smem + G::sK_n;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
    const int bh = blockIdx.x / nstates, s = blockIdx.x % nstates;
    const int n_chunks = (N + C - 1) / C;
    const int c0 = s * CPS, c1 = min(c0 + CPS, n_chunks);
    const T *Kh = K + (size_t)bh * N * D;
    const T *Vh = V + (size_t)bh * N * M;

    f32x4 acc[G::S_PER_WAVE];
#pragma unroll
    for (int i = 0; i < G::S_PER_WAVE; ++i) acc[i] = zero4();
    float z = 0.0f;

    Stage<T, C, D> stK;
    Stage<T, C, M> stV;
    if (c0 < c1) {
        stK.load(Kh, c0 * C, N, tid);
        stV.load(Vh, c0 * C, N, tid);
    }
    for (int c = c0; c < c1; ++c) {
        const int row0 = c * C;
        if constexpr (G::F32) {
            stK.template store_natural<true>(sKx, G::LQ, row0, N, tid);
            stV.template store_natural<false>(sVx, G::LV, row0, N, tid);
        } else {
            stK.template store_transposed<true, false>(sKx, G::LT, nullptr, 0, row0, N, tid);
            stV.template store_transposed<false, false>(sVx, G::LT, nullptr, 0, row0, N, tid);
        }
        __syncthreads();
        if (c + 1 < c1) {
            stK.load(Kh, row0 + C, N, tid);
            stV.load(Vh, row0 + C, N, tid);
        }
        state_update<T, D, M, C>(acc, sKx, sVx, w, g, l16);
        z = z_update<T, D, M, C>(z, sKx, tid);
        __syncthreads();
    }
    float *slot = ws + ((size_t)bh * (G_ + 1) + s) * G::E;
    state_to_global<T, D, M, C>(acc, z, slot, slot + D * M, w, g, l16, tid);
}

// ---------------------------------------------------------------------------
// Stage 3: outputs of one segment, from the exclusive prefix in its slot
// (causal) or from the total in slot G (non-causal).
// ---------------------------------------------------------------------------
template <typename T, int D, int M, int C, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void seg_output_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                              const T *__restrict__ V, float *__restrict__ out,
                                                              const float *__restrict__ ws, int N, int G_,
                                                              int CPS, float *__restrict__ S_out,
                                                              float *__restrict__ z_out) {
    using G = Cfg<T, D, M, C>;
    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[G::out_bytes];
    T *smem = reinterpret_cast<T *>(smem_raw);
    T *sQ = smem + G::oQ;
    T *sK = smem + G::oK;
    T *sV = smem + G::oV;   // fp32: V natural; bf16: V^T
    T *sKt = smem + G::oKt; // bf16 only
    T *sS = smem + G::oS;   // fp32: S natural; bf16: S^T
    float *sz = reinterpret_cast<float *>(smem_raw + ((G::nT_out * sizeof(T) + 15) / 16) * 16);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
    const int bh = blockIdx.x / G_, s = blockIdx.x % G_;
    const int n_chunks = (N + C - 1) / C;
    const int c0 = s * CPS, c1 = min(c0 + CPS, n_chunks);
    const T *Qh = Q + (size_t)bh * N * D;
    const T *Kh = K + (size_t)bh * N * D;
    const T *Vh = V + (size_t)bh * N * M;
    float *Oh = out + (size_t)bh * N * M;

    f32x4 acc[G::S_PER_WAVE];
    float z = 0.0f;
    if constexpr (CAUSAL) {
        if (s > 0) {
            state_from_global<T, D, M, C>(acc, z, ws + ((size_t)bh * (G_ + 1) + s) * G::E, w, g, l16, tid);
        } else {
#pragma unroll
            for (int i = 0; i < G::S_PER_WAVE; ++i) acc[i] = zero4();
        }
        state_to_lds<T, D, M, C>(acc, z, sS, sz, w, g, l16, tid);
    } else {
        const float *st = ws + ((size_t)bh * (G_ + 1) + G_) * G::E;
        for (int e = tid; e < D * M; e += kThreads) {
            const int d = e / M, m = e % M;
            if constexpr (G::F32)
                sS[d * G::LV + m] = st[e];
            else
                sS[m * G::LQ + d] = (bf16)st[e];
        }
        if (tid < D) sz[tid] = round_as<T>(st[D * M + tid]);
    }

    Stage<T, C, D> stQ, stK;
    Stage<T, C, M> stV;
    if (c0 < c1) {
        stQ.load(Qh, c0 * C, N, tid);
        if constexpr (CAUSAL) {
            stK.load(Kh, c0 * C, N, tid);
            stV.load(Vh, c0 * C, N, tid);
        }
    }
    const int rgrp = w % G::NWR, mgrp = w / G::NWR;

    for (int c = c0; c < c1; ++c) {
        const int row0 = c * C;
        stQ.template store_natural<true>(sQ, G::LQ, row0, N, tid);
        if constexpr (CAUSAL) {
            if constexpr (G::F32) {
                stK.template store_natural<true>(sK, G::LQ, row0, N, tid);
                stV.template store_natural<false>(sV, G::LV, row0, N, tid);
            } else {
                stK.template store_transposed<true, true>(sKt, G::LT, sK, G::LQ, row0, N, tid);
                stV.template store_transposed<false, false>(sV, G::LT, nullptr, 0, row0, N, tid);
            }
        }
        __syncthreads();
        if (c + 1 < c1) {
            stQ.load(Qh, row0 + C, N, tid);
            if constexpr (CAUSAL) {
                stK.load(Kh, row0 + C, N, tid);
                stV.load(Vh, row0 + C, N, tid);
            }
        }

        for (int rt = rgrp; rt < G::RT; rt += G::NWR) {
            const int qrow = rt * 16 + l16;
            f32x4 at[G::RT];
            float den = 0.0f;
            if constexpr (CAUSAL) {
#pragma unroll
                for (int kt = 0; kt < G::RT; ++kt) {
                    at[kt] = zero4();
                    if (kt <= rt) {
                        f32x4 a = zero4();
                        if constexpr (G::F32)
                            a = tile_dot_f32<D>(sK + (kt * 16 + l16) * G::LQ, 1, sQ + qrow * G::LQ, 1, g, a);
                        else
                            a = tile_dot_bf16<D>(sK + (kt * 16 + l16) * G::LQ, sQ + qrow * G::LQ, g, a);
                        // a[r] = A[query = rt*16 + l16][key = kt*16 + 4g + r]
                        if (kt == rt) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (4 * g + r > l16) a[r] = 0.0f;
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            a[r] = round_as<T>(a[r]);
                            den += a[r];
                        }
                        at[kt] = a;
                    }
                }
            }
            {
                const T *qr = sQ + qrow * G::LQ + g * (D / 4);
                const float *zr = sz + g * (D / 4);
#pragma unroll
                for (int j = 0; j < D / 4; ++j) den += to_f32(qr[j]) * zr[j];
            }
            den = sum_over_groups(den);
            const float inv = 1.0f / den;
            float inv_r[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) inv_r[r] = __shfl(inv, 4 * g + r, 64);

            for (int mt = mgrp; mt < G::MT; mt += G::NWM) {
                f32x4 o = zero4();
                if constexpr (CAUSAL) {
                    if constexpr (G::F32) {
#pragma unroll
                        for (int kt = 0; kt < G::RT; ++kt) {
                            if (kt <= rt) {
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    o = mma_f32(at[kt][r], sV[(kt * 16 + 4 * g + r) * G::LV + mt * 16 + l16], o);
                            }
                        }
                    } else if constexpr (G::RT == 1) {
                        bf16x4 a = {(bf16)at[0][0], (bf16)at[0][1], (bf16)at[0][2], (bf16)at[0][3]};
                        bf16x4 b = *reinterpret_cast<const bf16x4 *>(sV + (mt * 16 + l16) * G::LT + 4 * g);
                        o = mma_bf16_k16(a, b, o);
                    } else {
#pragma unroll
                        for (int p = 0; p < G::RT / 2; ++p) {
                            const int kt0 = 2 * p, kt1 = 2 * p + 1;
                            if (kt0 <= rt) {
                                const T *vrow = sV + (mt * 16 + l16) * G::LT;
                                bf16x4 b0 = *reinterpret_cast<const bf16x4 *>(vrow + kt0 * 16 + 4 * g);
                                bf16x4 b1 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
                                if (kt1 <= rt) b1 = *reinterpret_cast<const bf16x4 *>(vrow + kt1 * 16 + 4 * g);
                                bf16x8 a = {(bf16)at[kt0][0], (bf16)at[kt0][1], (bf16)at[kt0][2], (bf16)at[kt0][3],
                                            (bf16)at[kt1][0], (bf16)at[kt1][1], (bf16)at[kt1][2], (bf16)at[kt1][3]};
                                bf16x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                                o = mma_bf16_k32(a, b, o);
                            }
                        }
                    }
                }
                // inter-chunk term phi(Q_c) S
                if constexpr (G::F32)
                    o = tile_dot_f32<D>(sQ + qrow * G::LQ, 1, sS + mt * 16 + l16, G::LV, g, o);
                else
                    o = tile_dot_bf16<D>(sQ + qrow * G::LQ, sS + (mt * 16 + l16) * G::LQ, g, o);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int grow = row0 + rt * 16 + 4 * g + r;
                    if (grow < N) Oh[(size_t)grow * M + mt * 16 + l16] = o[r] * inv_r[r];
                }
            }
        }

        if constexpr (CAUSAL) {
            state_update<T, D, M, C>(acc, G::F32 ? sK : sKt, sV, w, g, l16);
            z = z_update<T, D, M, C>(z, G::F32 ? sK : sKt, tid);
        }
        __syncthreads();
        if constexpr (CAUSAL) state_to_lds<T, D, M, C>(acc, z, sS, sz, w, g, l16, tid);
    }

    if constexpr (CAUSAL) {
        if (S_out != nullptr && s == G_ - 1)
            state_to_global<T, D, M, C>(acc, z, S_out + (size_t)bh * D * M, z_out + (size_t)bh * D, w, g, l16, tid);
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers (instantiated per element type in la_prefill_*.hip).
// ---------------------------------------------------------------------------
template <typename T, int D, int M, int C>
hipError_t run_states(const void *K, const void *V, float *ws, int BH, int N, int G_, int CPS, int nstates,
                      hipStream_t stream) {
    using G = Cfg<T, D, M, C>;
    if constexpr (!G::fits) {
        return hipErrorInvalidValue;
    } else {
        if (nstates <= 0 || BH <= 0) return hipSuccess;
        hipLaunchKernelGGL((seg_state_kernel<T, D, M, C>), dim3((unsigned)(BH * nstates)), dim3(kThreads), 0, stream,
                           (const T *)K, (const T *)V, ws, N, G_, CPS, nstates);
        return hipGetLastError();
    }
}

template <typename T, int D, int M, int C>
hipError_t run_outputs(const void *Q, const void *K, const void *V, float *out, const float *ws, int BH, int N,
                       int G_, int CPS, int causal, float *S_out, float *z_out, hipStream_t stream) {
    using G = Cfg<T, D, M, C>;
    if constexpr (!G::fits) {
        return hipErrorInvalidValue;
    } else {
        if (BH <= 0 || G_ <= 0) return hipSuccess;
        const dim3 grid((unsigned)(BH * G_)), block(kThreads);
        if (causal)
            hipLaunchKernelGGL((seg_output_kernel<T, D, M, C, true>), grid, block, 0, stream, (const T *)Q,
                               (const T *)K, (const T *)V, out, ws, N, G_, CPS, S_out, z_out);
        else
            hipLaunchKernelGGL((seg_output_kernel<T, D, M, C, false>), grid, block, 0, stream, (const T *)Q,
                               (const T *)K, (const T *)V, out, ws, N, G_, CPS, S_out, z_out);
        return hipGetLastError();
    }
}

}  // namespace la
