// Gradients of causal kernelized linear attention (training half of the
// parallel mode).
//
// Page "Transformers are RNNs" (Katharopoulos et al., 2020), Proposed method:
// the gradients are computed in linear time with running sums, like the forward
// pass.  With g_i = phi(q_i), f_j = phi(k_j), S_i, z_i the forward sums,
// den_i = g_i . z_i and out_i the forward output, the chain rule through
// out_i = g_i^T S_i / den_i gives
//   r_i = dout_i / den_i,   c_i = -(dout_i . out_i) / den_i
//   dg_i = S_i r_i + c_i z_i                         (forward sums, j <= i)
//   df_j = R_j v_j + w_j,   dv_j = R_j^T f_j          (reverse sums, i >= j)
// with R_j = sum_{i>=j} g_i r_i^T and w_j = sum_{i>=j} c_i g_i;
// dq = dg * phi'(q), dk = df * phi'(k), and phi'(x) = min(phi(x), 1).
// Inputs that already hold features (PHI = false, for example random features
// formed by the feature-map kernel) get dg and df themselves: the gradients with
// respect to the features, which the feature map's own backward carries on.
//
// Chunked form, chunk c of C rows, masks keep i >= j:
//   dG_c = tril(R_c V_c^T + c 1^T) F_c + R_c S_prev^T + c z_prev^T
//   dF_c = triu(V_c R_c^T + 1 c^T) G_c + V_c R_next^T + 1 w_next^T
//   dV_c = triu(F_c G_c^T) R_c + F_c R_next
// (S_prev, z_prev: sums over earlier positions; R_next, w_next: over later ones.)
//
// Launch sequence (la_backward_chunked): forward segment states and their
// exclusive scan (the forward's stage kernels), bwd_dq_kernel (walks each
// segment forward: den, dQ, and the segment's reverse state), the reverse
// exclusive scan of those states, bwd_dkv_kernel (walks each segment backward:
// dK, dV).  Every contraction runs on fp32 MFMA (v_mfma_f32_16x16x4_f32);
// bf16 inputs are widened when staged.  Four wavefronts per workgroup; the
// query-side state is held transposed (lane: d = l16, m = 4g + r) so that it
// is directly the MFMA operand of R S^T.
#pragma once

#include "la_device.hpp"

namespace la {

constexpr int kBwdChunk = 32;
constexpr int kBwdThreads = 256;
constexpr int kBwdWaves = 4;

template <int D, int M>
struct BwdCfg {
    static constexpr int C = kBwdChunk;
    static constexpr int RT = C / 16, DT = D / 16, MT = M / 16;
    static constexpr int DTW = (DT + kBwdWaves - 1) / kBwdWaves;  // d-tiles per wavefront
    static constexpr int MTW = (MT + kBwdWaves - 1) / kBwdWaves;  // m-tiles per wavefront
    static constexpr int LD = D + 4, LM = M + 4, LC = C + 4;      // padded row lengths (floats)
    static constexpr int oG = 0;
    static constexpr int oF = oG + C * LD;
    static constexpr int oV = oF + C * LD;
    static constexpr int oO = oV + C * LM;
    static constexpr int oR = oO + C * LM;   // dout, then r = dout / den in place
    static constexpr int oP = oR + C * LM;   // [C][LC]
    static constexpr int oP2 = oP + C * LC;  // [C][LC]
    static constexpr int oZ = oP2 + C * LC;  // z_prev or w_next [D]
    static constexpr int oDen = oZ + D;      // [C]
    static constexpr int oCc = oDen + C;     // c_i [C]
    static constexpr int oDenp = oCc + C;    // [RT][C]
    static constexpr int oQz = oDenp + RT * C;
    static constexpr int NCS = kBwdThreads / D < C ? kBwdThreads / D : C;  // column-sum groups
    static constexpr int oCol = oQz + C;     // [2][NCS][D] column-sum partials
    static constexpr int nF = oCol + 2 * NCS * D;
    static constexpr size_t bytes = (size_t)nF * 4;
    static_assert(C % NCS == 0, "column-sum split");
};

// A C x W tile of a [N][W] head matrix (element type T), staged as fp32 into LDS
// rows of length ld in two steps: load() issues every global load of the tile
// into registers (rows at or beyond N reload row N - 1), store() writes it to
// LDS (through phi when asked; rows at or beyond N as zeros).  Loading the next
// chunk's tiles before the current chunk's arithmetic keeps the loads in flight
// meanwhile; a load-then-store loop per element instead waits for each load.
template <typename T, int C, int W>
struct BwdTile {
    static constexpr int NV = W / 4;
    static constexpr int PER = (C * NV + kBwdThreads - 1) / kBwdThreads;
    f32x4 x[PER];
    __device__ __forceinline__ void load(const T *__restrict__ src, int row0, int N, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + i * kBwdThreads;
            if (PER * kBwdThreads == C * NV || e < C * NV) {
                const int row = e / NV, cv = e % NV;
                const T *p = src + (size_t)min(row0 + row, N - 1) * W + cv * 4;
                if constexpr (std::is_same<T, float>::value) {
                    x[i] = *reinterpret_cast<const f32x4 *>(p);
                } else {
                    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
                    x[i] = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
                }
            }
        }
    }
    template <bool PHI>
    __device__ __forceinline__ void store(float *dst, int ld, int row0, int N, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + i * kBwdThreads;
            if (PER * kBwdThreads == C * NV || e < C * NV) {
                const int row = e / NV, cv = e % NV;
                f32x4 v = x[i];
                if (PHI) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = phi(v[j]);
                }
                if (row0 + row >= N) v = zero4();
                *reinterpret_cast<f32x4 *>(dst + row * ld + cv * 4) = v;
            }
        }
    }
};

// The five tiles of a chunk (q, k, v, out, dout).
template <typename T, int C, int D, int M>
struct BwdChunk {
    BwdTile<T, C, D> q, k;
    BwdTile<T, C, M> v;
    BwdTile<float, C, M> o, dout;
    __device__ __forceinline__ void load(const T *Qh, const T *Kh, const T *Vh, const float *Oh, const float *dOh,
                                         int row0, int N, int tid) {
        q.load(Qh, row0, N, tid);
        k.load(Kh, row0, N, tid);
        v.load(Vh, row0, N, tid);
        o.load(Oh, row0, N, tid);
        dout.load(dOh, row0, N, tid);
    }
};

template <int D, int M>
struct BwdEngine {
    using G = BwdCfg<D, M>;
    static constexpr int C = G::C, RT = G::RT, DT = G::DT, MT = G::MT, DTW = G::DTW, MTW = G::MTW;
    float *sG, *sF, *sV, *sO, *sR, *sP, *sP2, *sZ, *sDen, *sCc, *sDenp, *sQz, *sCol;
    int tid, lane, w, g, l16;

    __device__ __forceinline__ explicit BwdEngine(float *smem) {
        sG = smem + G::oG;
        sF = smem + G::oF;
        sV = smem + G::oV;
        sO = smem + G::oO;
        sR = smem + G::oR;
        sP = smem + G::oP;
        sP2 = smem + G::oP2;
        sZ = smem + G::oZ;
        sDen = smem + G::oDen;
        sCc = smem + G::oCc;
        sDenp = smem + G::oDenp;
        sQz = smem + G::oQz;
        sCol = smem + G::oCol;
        tid = threadIdx.x;
        lane = tid & 63;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
        g = lane >> 4;
        l16 = lane & 15;
    }
    __device__ __forceinline__ bool owns_d(int i) const { return w + kBwdWaves * i < DT; }
    __device__ __forceinline__ int dtile(int i) const { return w + kBwdWaves * i; }
    __device__ __forceinline__ bool owns_m(int i) const { return w + kBwdWaves * i < MT; }
    __device__ __forceinline__ int mtile(int i) const { return w + kBwdWaves * i; }

    // Masked C x C product tiles: out[a][b] = sum_k X[a][k] Y[b][k] over K columns,
    // kept where (UPPER ? b >= a : b <= a), plus add_a[a] and add_b[b] (if given)
    // on kept entries; written to dst[a][b].  Row tiles (at, bt) of the kept triangle are
    // shared out over the wavefronts.  Rows of X and Y are read as f32x4 (the
    // contraction index d = g*(K/4) + j is contiguous per lane).
    template <int K, bool UPPER>
    __device__ __forceinline__ void tri_tiles(const float *X, int ldx, const float *Y, int ldy, const float *add_b,
                                              float *dst, const float *add_a = nullptr) const {
        constexpr int NA = RT * (RT + 1) / 2;
        for (int t = w; t < NA; t += kBwdWaves) {
            int hi = 0;
            while ((hi + 1) * (hi + 2) / 2 <= t) ++hi;
            const int lo = t - hi * (hi + 1) / 2;  // lo <= hi
            const int at = UPPER ? lo : hi, bt = UPPER ? hi : lo;
            // result tile computed transposed: acc[r] = out[a = at*16 + l16... ] -- see below
            f32x4 acc = zero4();
            const float *yrow = Y + (bt * 16 + l16) * ldy;  // A operand rows: b
            const float *xrow = X + (at * 16 + l16) * ldx;  // B operand columns: a
#pragma unroll
            for (int j4 = 0; j4 < K / 16; ++j4) {
                const f32x4 yv = *reinterpret_cast<const f32x4 *>(yrow + g * (K / 4) + 4 * j4);
                const f32x4 xv = *reinterpret_cast<const f32x4 *>(xrow + g * (K / 4) + 4 * j4);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc = mma_f32(yv[j], xv[j], acc);
            }
            // acc[r] = out[a = at*16 + l16][b = bt*16 + 4g + r]
            const int a = at * 16 + l16;
            const float ya = add_a ? add_a[a] : 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int b = bt * 16 + 4 * g + r;
                const bool keep = UPPER ? (b >= a) : (b <= a);
                float v = acc[r] + ya + (add_b ? add_b[b] : 0.0f);
                acc[r] = keep ? v : 0.0f;
            }
            *reinterpret_cast<f32x4 *>(dst + a * G::LC + bt * 16 + 4 * g) = acc;
        }
    }

    // zero the tiles tri_tiles never writes (the other triangle), once per kernel
    __device__ __forceinline__ void clear_tiles() const {
        for (int e = tid; e < 2 * C * G::LC; e += kBwdThreads) sP[e] = 0.0f;  // sP and sP2 are adjacent
    }

    // per-thread partial column sums of (weights[row] *) rows of X (C x D) -> part[q][d]
    __device__ __forceinline__ void col_partials(const float *X, const float *weights, float *part) const {
        constexpr int NCS = G::NCS, ROWS = C / NCS;
        const int q = tid / D, d = tid % D;
        if (q < NCS) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < ROWS; ++i) {
                const int row = q * ROWS + i;
                s += (weights ? weights[row] : 1.0f) * X[row * G::LD + d];
            }
            part[q * D + d] = s;
        }
    }
    __device__ __forceinline__ float col_total(const float *part) const {  // thread tid < D
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < G::NCS; ++q) s += part[q * D + tid];
        return s;
    }

    // dot products of rows: out[i] = X[i] . Y[i] over K columns (TPR threads per row)
    template <int K>
    __device__ __forceinline__ void row_dots(const float *X, int ldx, const float *Y, int ldy, float *out) const {
        constexpr int TPR = kBwdThreads / C;  // 8 threads per row, each K/8 contiguous columns
        constexpr int EPT = K / TPR;
        const int i = tid / TPR, p = tid % TPR;
        const float *x = X + i * ldx + p * EPT, *y = Y + i * ldy + p * EPT;
        float s = 0.0f;
        if constexpr (EPT % 4 == 0) {
#pragma unroll
            for (int v = 0; v < EPT / 4; ++v) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(x + 4 * v);
                const f32x4 b = *reinterpret_cast<const f32x4 *>(y + 4 * v);
                s += (a[0] * b[0] + a[1] * b[1]) + (a[2] * b[2] + a[3] * b[3]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < EPT; ++k) s += x[k] * y[k];
        }
        static_assert(TPR <= 16, "threads of a row within one 16-lane row");
        s = row_group_sum<TPR>(s);
        if (p == 0) out[i] = s;
    }
};

// Workspace slot layout of the states exchanged between the kernels: the
// forward stage format, [D][M] row major then z[D] (E = D*M + D floats).

// ---------------------------------------------------------------------------
// dQ: walk the segment's chunks forward from (S_prev, z_prev).
// ---------------------------------------------------------------------------
template <typename T, int D, int M, bool PHI = true>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                             const T *__restrict__ V, const float *__restrict__ O,
                                                             const float *__restrict__ dO,
                                                             const float *__restrict__ fwd_ws, float *rev_ws,
                                                             float *__restrict__ den_out, float *__restrict__ dQ,
                                                             int N, int G_, int CPS) {
    using Gc = BwdCfg<D, M>;
    using En = BwdEngine<D, M>;
    constexpr int C = Gc::C, E = D * M + D;
    __shared__ __attribute__((aligned(16))) float smem[Gc::nF];
    En e(smem);
    const int tid = e.tid;
    const int bh = blockIdx.x / G_, s = blockIdx.x % G_;
    const int n_chunks = (N + C - 1) / C;
    const int c0 = s * CPS, c1 = min(c0 + CPS, n_chunks);
    const size_t hq = (size_t)bh * N * D, hv = (size_t)bh * N * M;

    // S^T tiles: St[i][mt][r] = S[d = dtile(i)*16 + l16][m = mt*16 + 4g + r]
    f32x4 St[Gc::DTW][Gc::MT];
    f32x4 Rs[Gc::DTW][Gc::MT];  // the segment's reverse state, same layout
#pragma unroll
    for (int i = 0; i < Gc::DTW; ++i)
#pragma unroll
        for (int mt = 0; mt < Gc::MT; ++mt) {
            St[i][mt] = zero4();
            Rs[i][mt] = zero4();
        }
    float zprev = 0.0f, wseg = 0.0f;  // thread tid < D: element tid
    const float *pre = fwd_ws + ((size_t)bh * (G_ + 1) + s) * E;
    if (s > 0) {
#pragma unroll
        for (int i = 0; i < Gc::DTW; ++i) {
            if (!e.owns_d(i)) continue;
            const int d = e.dtile(i) * 16 + e.l16;
#pragma unroll
            for (int mt = 0; mt < Gc::MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) St[i][mt][r] = pre[d * M + mt * 16 + 4 * e.g + r];
        }
        if (tid < D) zprev = pre[D * M + tid];
    }
    e.clear_tiles();

    // loads one chunk ahead, unconditional (the index clamped to the last chunk) so
    // that the compiler's wait counts stay exact
    BwdChunk<T, C, D, M> ld;
    ld.load(Q + hq, K + hq, V + hv, O + hv, dO + hv, c0 * C, N, tid);
    for (int c = c0; c < c1; ++c) {
        const int row0 = c * C;
        __syncthreads();
        ld.q.template store<PHI>(e.sG, Gc::LD, row0, N, tid);
        ld.k.template store<PHI>(e.sF, Gc::LD, row0, N, tid);
        ld.v.template store<false>(e.sV, Gc::LM, row0, N, tid);
        ld.o.template store<false>(e.sO, Gc::LM, row0, N, tid);
        ld.dout.template store<false>(e.sR, Gc::LM, row0, N, tid);
        if (tid < D) e.sZ[tid] = zprev;
        __syncthreads();
        ld.load(Q + hq, K + hq, V + hv, O + hv, dO + hv, min(c + 1, c1 - 1) * C, N, tid);
        // den_i = rowsum(tril(G F^T)) + g_i . z_prev ; (dout . out)_i
        e.template tri_tiles<D, false>(e.sG, Gc::LD, e.sF, Gc::LD, nullptr, e.sP);
        e.template row_dots<D>(e.sG, Gc::LD, e.sZ, 0, e.sQz);
        e.template row_dots<M>(e.sR, Gc::LM, e.sO, Gc::LM, e.sCc);
        __syncthreads();
        if (tid < C) {
            // row sum of tril(A): the tile rows as 16-byte reads
            float den = e.sQz[tid];
#pragma unroll
            for (int j4 = 0; j4 < C / 4; ++j4) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(e.sP + tid * Gc::LC + 4 * j4);
                den += (a[0] + a[1]) + (a[2] + a[3]);
            }
            if (row0 + tid >= N) den = 1.0f;  // padding rows: r = c = 0
            const float inv = 1.0f / den;
            e.sDen[tid] = inv;  // 1 / den from here on
            e.sCc[tid] = -e.sCc[tid] * inv;
            if (row0 + tid < N) den_out[(size_t)bh * N + row0 + tid] = den;
        }
        __syncthreads();
        for (int x = tid; x < C * M / 4; x += kBwdThreads) {
            const int i = x / (M / 4), m4 = x % (M / 4);
            f32x4 *p = reinterpret_cast<f32x4 *>(e.sR + i * Gc::LM + 4 * m4);
            *p = *p * e.sDen[i];
        }
        __syncthreads();
        // B = tril(R V^T + c 1^T): B[i][j] = r_i . v_j + c_i for j <= i (stored [i][j])
        e.template tri_tiles<M, false>(e.sR, Gc::LM, e.sV, Gc::LM, nullptr, e.sP, e.sCc);
        __syncthreads();
        // dG^T tiles for the own d-tiles, rows i of the chunk
#pragma unroll
        for (int ii = 0; ii < Gc::DTW; ++ii) {
            if (!e.owns_d(ii)) continue;
            const int dt = e.dtile(ii);
#pragma unroll
            for (int rt = 0; rt < Gc::RT; ++rt) {
                f32x4 acc = zero4();
                const int irow = rt * 16 + e.l16;
                // B F: contraction over keys j (lane group g owns keys g*8 .. g*8+7)
                const float *brow = e.sP + irow * Gc::LC + e.g * (C / 4);
#pragma unroll
                for (int j4 = 0; j4 < C / 16; ++j4) {
                    const f32x4 bv = *reinterpret_cast<const f32x4 *>(brow + 4 * j4);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int j = e.g * (C / 4) + 4 * j4 + jj;
                        acc = mma_f32(e.sF[j * Gc::LD + dt * 16 + e.l16], bv[jj], acc);
                    }
                }
                // R S^T: contraction over m, S^T from registers
#pragma unroll
                for (int mt = 0; mt < Gc::MT; ++mt) {
                    const f32x4 rv = *reinterpret_cast<const f32x4 *>(e.sR + irow * Gc::LM + mt * 16 + 4 * e.g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc = mma_f32(St[ii][mt][r], rv[r], acc);
                }
                // acc[r] = dG[i = irow][d = dt*16 + 4g + r]; + c_i z_prev[d]; times phi'(q) = min(phi(q), 1)
                const int i = irow, grow = row0 + i;
                const float ci = e.sCc[i];
                const f32x4 gq = *reinterpret_cast<const f32x4 *>(e.sG + i * Gc::LD + dt * 16 + 4 * e.g);
                f32x4 outv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float dg = acc[r] + ci * e.sZ[dt * 16 + 4 * e.g + r];
                    outv[r] = PHI ? dg * fminf(gq[r], 1.0f) : dg;
                }
                if (grow < N) *reinterpret_cast<f32x4 *>(dQ + hq + (size_t)grow * D + dt * 16 + 4 * e.g) = outv;
            }
        }
        // state updates: S^T += V^T F ; Rs^T += R^T G (rows m = 4g + r, columns d = l16)
#pragma unroll
        for (int ks = 0; ks < C / 4; ++ks) {
            const int j = 4 * ks + e.g;
#pragma unroll
            for (int ii = 0; ii < Gc::DTW; ++ii) {
                if (!e.owns_d(ii)) continue;
                const int dcol = e.dtile(ii) * 16 + e.l16;
                const float fb = e.sF[j * Gc::LD + dcol];
                const float gb = e.sG[j * Gc::LD + dcol];
#pragma unroll
                for (int mt = 0; mt < Gc::MT; ++mt) {
                    St[ii][mt] = mma_f32(e.sV[j * Gc::LM + mt * 16 + e.l16], fb, St[ii][mt]);
                    Rs[ii][mt] = mma_f32(e.sR[j * Gc::LM + mt * 16 + e.l16], gb, Rs[ii][mt]);
                }
            }
        }
        // z_prev += colsum F ; w_seg += colsum (c * G)
        e.col_partials(e.sF, nullptr, e.sCol);
        e.col_partials(e.sG, e.sCc, e.sCol + Gc::NCS * D);
        __syncthreads();
        if (tid < D) {
            zprev += e.col_total(e.sCol);
            wseg += e.col_total(e.sCol + Gc::NCS * D);
        }
    }
    // the segment's reverse state -> rev_ws slot s ([D][M] then w[D])
    float *slot = rev_ws + ((size_t)bh * (G_ + 1) + s) * E;
#pragma unroll
    for (int ii = 0; ii < Gc::DTW; ++ii) {
        if (!e.owns_d(ii)) continue;
        const int d = e.dtile(ii) * 16 + e.l16;
#pragma unroll
        for (int mt = 0; mt < Gc::MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) slot[d * M + mt * 16 + 4 * e.g + r] = Rs[ii][mt][r];
    }
    if (tid < D) slot[D * M + tid] = wseg;
}

// ---------------------------------------------------------------------------
// dK, dV: walk the segment's chunks backward from (R_next, w_next).
// ---------------------------------------------------------------------------
template <typename T, int D, int M, bool PHI = true>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dkv_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                              const T *__restrict__ V, const float *__restrict__ O,
                                                              const float *__restrict__ dO,
                                                              const float *__restrict__ rev_ws,
                                                              const float *__restrict__ den_in,
                                                              float *__restrict__ dK, float *__restrict__ dV, int N,
                                                              int G_, int CPS) {
    using Gc = BwdCfg<D, M>;
    using En = BwdEngine<D, M>;
    constexpr int C = Gc::C, E = D * M + D;
    __shared__ __attribute__((aligned(16))) float smem[Gc::nF];
    En e(smem);
    const int tid = e.tid;
    const int bh = blockIdx.x / G_, s = blockIdx.x % G_;
    const int n_chunks = (N + C - 1) / C;
    const int c0 = s * CPS, c1 = min(c0 + CPS, n_chunks);
    const size_t hq = (size_t)bh * N * D, hv = (size_t)bh * N * M;

    // RnT[i][mt][r] = R_next[d = dtile(i)*16 + l16][m = mt*16 + 4g + r]   (for dF)
    // Rn[i][dt][r]  = R_next[d = dt*16 + 4g + r][m = mtile(i)*16 + l16]   (for dV)
    f32x4 RnT[Gc::DTW][Gc::MT];
    f32x4 Rn[Gc::MTW][Gc::DT];
#pragma unroll
    for (int i = 0; i < Gc::DTW; ++i)
#pragma unroll
        for (int mt = 0; mt < Gc::MT; ++mt) RnT[i][mt] = zero4();
#pragma unroll
    for (int i = 0; i < Gc::MTW; ++i)
#pragma unroll
        for (int dt = 0; dt < Gc::DT; ++dt) Rn[i][dt] = zero4();
    float wnext = 0.0f;
    if (s < G_ - 1) {
        const float *suf = rev_ws + ((size_t)bh * (G_ + 1) + s) * E;  // sum over later segments
#pragma unroll
        for (int i = 0; i < Gc::DTW; ++i) {
            if (!e.owns_d(i)) continue;
            const int d = e.dtile(i) * 16 + e.l16;
#pragma unroll
            for (int mt = 0; mt < Gc::MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) RnT[i][mt][r] = suf[d * M + mt * 16 + 4 * e.g + r];
        }
#pragma unroll
        for (int i = 0; i < Gc::MTW; ++i) {
            if (!e.owns_m(i)) continue;
            const int m = e.mtile(i) * 16 + e.l16;
#pragma unroll
            for (int dt = 0; dt < Gc::DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) Rn[i][dt][r] = suf[(dt * 16 + 4 * e.g + r) * M + m];
        }
        if (tid < D) wnext = suf[D * M + tid];
    }
    e.clear_tiles();

    // loads one chunk ahead (walking backward), unconditional (clamped to the first chunk)
    BwdChunk<T, C, D, M> ld;
    ld.load(Q + hq, K + hq, V + hv, O + hv, dO + hv, (c1 - 1) * C, N, tid);
    for (int c = c1 - 1; c >= c0; --c) {
        const int row0 = c * C;
        __syncthreads();
        ld.q.template store<PHI>(e.sG, Gc::LD, row0, N, tid);
        ld.k.template store<PHI>(e.sF, Gc::LD, row0, N, tid);
        ld.v.template store<false>(e.sV, Gc::LM, row0, N, tid);
        ld.o.template store<false>(e.sO, Gc::LM, row0, N, tid);
        ld.dout.template store<false>(e.sR, Gc::LM, row0, N, tid);
        if (tid < D) e.sZ[tid] = wnext;
        if (tid < C) e.sDen[tid] = row0 + tid < N ? den_in[(size_t)bh * N + row0 + tid] : 1.0f;
        __syncthreads();
        ld.load(Q + hq, K + hq, V + hv, O + hv, dO + hv, max(c - 1, c0) * C, N, tid);
        e.template row_dots<M>(e.sR, Gc::LM, e.sO, Gc::LM, e.sCc);
        __syncthreads();
        if (tid < C) e.sCc[tid] = -e.sCc[tid] / e.sDen[tid];
        for (int x = tid; x < C * M / 4; x += kBwdThreads) {
            const int i = x / (M / 4), m4 = x % (M / 4);
            f32x4 *p = reinterpret_cast<f32x4 *>(e.sR + i * Gc::LM + 4 * m4);
            *p = *p * (1.0f / e.sDen[i]);
        }
        __syncthreads();
        // P[j][i] = v_j . r_i + c_i (i >= j);  P2[j][i] = f_j . g_i (i >= j)
        e.template tri_tiles<M, true>(e.sV, Gc::LM, e.sR, Gc::LM, e.sCc, e.sP);
        e.template tri_tiles<D, true>(e.sF, Gc::LD, e.sG, Gc::LD, nullptr, e.sP2);
        __syncthreads();
        // dF^T tiles for the own d-tiles
#pragma unroll
        for (int ii = 0; ii < Gc::DTW; ++ii) {
            if (!e.owns_d(ii)) continue;
            const int dt = e.dtile(ii);
#pragma unroll
            for (int jt = 0; jt < Gc::RT; ++jt) {
                f32x4 acc = zero4();
                const int jrow = jt * 16 + e.l16;
                const float *prow = e.sP + jrow * Gc::LC + e.g * (C / 4);
#pragma unroll
                for (int i4 = 0; i4 < C / 16; ++i4) {
                    const f32x4 pv = *reinterpret_cast<const f32x4 *>(prow + 4 * i4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int i = e.g * (C / 4) + 4 * i4 + q;
                        acc = mma_f32(e.sG[i * Gc::LD + dt * 16 + e.l16], pv[q], acc);
                    }
                }
#pragma unroll
                for (int mt = 0; mt < Gc::MT; ++mt) {
                    const f32x4 vv = *reinterpret_cast<const f32x4 *>(e.sV + jrow * Gc::LM + mt * 16 + 4 * e.g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc = mma_f32(RnT[ii][mt][r], vv[r], acc);
                }
                // acc[r] = dF[j = jrow][d = dt*16 + 4g + r]; + w_next[d]; times phi'(k) = min(phi(k), 1)
                const int grow = row0 + jrow;
                const f32x4 fk = *reinterpret_cast<const f32x4 *>(e.sF + jrow * Gc::LD + dt * 16 + 4 * e.g);
                f32x4 outv;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    outv[r] = (acc[r] + e.sZ[dt * 16 + 4 * e.g + r]) * (PHI ? fminf(fk[r], 1.0f) : 1.0f);
                if (grow < N) *reinterpret_cast<f32x4 *>(dK + hq + (size_t)grow * D + dt * 16 + 4 * e.g) = outv;
            }
        }
        // dV^T tiles for the own m-tiles
#pragma unroll
        for (int ii = 0; ii < Gc::MTW; ++ii) {
            if (!e.owns_m(ii)) continue;
            const int mt = e.mtile(ii);
#pragma unroll
            for (int jt = 0; jt < Gc::RT; ++jt) {
                f32x4 acc = zero4();
                const int jrow = jt * 16 + e.l16;
                const float *prow = e.sP2 + jrow * Gc::LC + e.g * (C / 4);
#pragma unroll
                for (int i4 = 0; i4 < C / 16; ++i4) {
                    const f32x4 pv = *reinterpret_cast<const f32x4 *>(prow + 4 * i4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int i = e.g * (C / 4) + 4 * i4 + q;
                        acc = mma_f32(e.sR[i * Gc::LM + mt * 16 + e.l16], pv[q], acc);
                    }
                }
#pragma unroll
                for (int dt = 0; dt < Gc::DT; ++dt) {
                    const f32x4 fv = *reinterpret_cast<const f32x4 *>(e.sF + jrow * Gc::LD + dt * 16 + 4 * e.g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc = mma_f32(Rn[ii][dt][r], fv[r], acc);
                }
                const int grow = row0 + jrow;
                if (grow < N) *reinterpret_cast<f32x4 *>(dV + hv + (size_t)grow * M + mt * 16 + 4 * e.g) = acc;
            }
        }
        // state updates: R_next += G^T R (both layouts); w_next += colsum(c * G)
#pragma unroll
        for (int ks = 0; ks < C / 4; ++ks) {
            const int i = 4 * ks + e.g;
#pragma unroll
            for (int ii = 0; ii < Gc::DTW; ++ii) {
                if (!e.owns_d(ii)) continue;
                const float gb = e.sG[i * Gc::LD + e.dtile(ii) * 16 + e.l16];
#pragma unroll
                for (int mt = 0; mt < Gc::MT; ++mt)
                    RnT[ii][mt] = mma_f32(e.sR[i * Gc::LM + mt * 16 + e.l16], gb, RnT[ii][mt]);
            }
#pragma unroll
            for (int ii = 0; ii < Gc::MTW; ++ii) {
                if (!e.owns_m(ii)) continue;
                const float rb = e.sR[i * Gc::LM + e.mtile(ii) * 16 + e.l16];
#pragma unroll
                for (int dt = 0; dt < Gc::DT; ++dt)
                    Rn[ii][dt] = mma_f32(e.sG[i * Gc::LD + dt * 16 + e.l16], rb, Rn[ii][dt]);
            }
        }
        e.col_partials(e.sG, e.sCc, e.sCol);
        __syncthreads();
        if (tid < D) wnext += e.col_total(e.sCol);
    }
}

// Reverse exclusive scan over segments: slot s <- sum of slots s+1 .. G-1 (per head).
// One thread per state element of one head; grid (ceil(E / 256), BH).
__global__ __launch_bounds__(256) void bwd_rev_scan_kernel(float *ws, int E, int G_) {
    const int x = blockIdx.x * 256 + threadIdx.x;
    if (x >= E) return;
    float *h = ws + (size_t)blockIdx.y * (G_ + 1) * E;
    float acc = 0.0f;
    // kScanBatch slots loaded before any is overwritten (one round trip per batch)
    for (int s1 = G_ - 1; s1 >= 0; s1 -= kScanBatch) {
        float v[kScanBatch];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) v[j] = s1 - j >= 0 ? h[(size_t)(s1 - j) * E + x] : 0.0f;
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) {
            if (s1 - j >= 0) {
                h[(size_t)(s1 - j) * E + x] = acc;
                acc += v[j];
            }
        }
    }
    h[(size_t)G_ * E + x] = acc;  // total
}

template <typename T, int D, int M, bool PHI = true>
hipError_t run_bwd_dq(const void *Q, const void *K, const void *V, const float *O, const float *dO,
                      const float *fwd_ws, float *rev_ws, float *den, float *dQ, int BH, int N, int G_, int CPS,
                      hipStream_t stream) {
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, M, PHI>), dim3((unsigned)(BH * G_)), dim3(kBwdThreads), 0, stream,
                       (const T *)Q, (const T *)K, (const T *)V, O, dO, fwd_ws, rev_ws, den, dQ, N, G_, CPS);
    return hipGetLastError();
}

template <typename T, int D, int M, bool PHI = true>
hipError_t run_bwd_dkv(const void *Q, const void *K, const void *V, const float *O, const float *dO,
                       const float *rev_ws, const float *den, float *dK, float *dV, int BH, int N, int G_, int CPS,
                       hipStream_t stream) {
    hipLaunchKernelGGL((bwd_dkv_kernel<T, D, M, PHI>), dim3((unsigned)(BH * G_)), dim3(kBwdThreads), 0, stream,
                       (const T *)Q, (const T *)K, (const T *)V, O, dO, rev_ws, den, dK, dV, N, G_, CPS);
    return hipGetLastError();
}

}  // namespace la
