// Parallel (prefill) mode of causal kernelized linear attention.
//
// Page "Transformers are RNNs" (Katharopoulos et al., 2020), Proposed method:
// attention with the similarity phi(q)^T phi(k) is rewritten by associativity as
// phi(Q) (phi(K)^T V); causal masking is kept by the cumulative sums S_i, Z_i.
// Each head's sequence is cut into chunks of C positions and the chunks into
// segments of whole chunks.  For a chunk c with the state (S, z) of all
// earlier positions:
//   A   = tril(phi(Q_c) phi(K_c)^T)               (C x C, diagonal kept)
//   num = A V_c + phi(Q_c) S                      (C x M)
//   den = rowsum(A) + phi(Q_c) z                  (C)
//   out = num / den
//   S  += phi(K_c)^T V_c ;  z += colsum(phi(K_c))
// A workgroup owns one segment.  In the two-phase fused kernel, phase A sums
// the segment's state; the states are chained across segments by an
// exclusive prefix (published per segment, decoupled look-back); phase B
// walks the segment's chunks from the prefix and writes the outputs.  The
// one-pass kernel (segments of at most four chunks) reads the segment once and
// applies the prefix after the look-back.
//
// Work split inside a workgroup of NW wavefronts (8 when M = 128, else 4):
// wavefront w owns the output / state columns m-tiles {w, w+NW, ...}.  It
// keeps S[:, its m-tiles] in MFMA accumulators,
// updates them (phi(K)^T V) and reads them out (phi(Q) S) straight from
// registers; the masked C x C matrix A is computed once per chunk (tiles
// shared out over the wavefronts) and passed through LDS.
//
// LDS (element type T = float or bf16):
//   fp32: phi(Q) [C][D+p]   phi(K) [C][D+p]   V [C][M+p]   A [C][C+p]
//   bf16: phi(Q) [C][D]     phi(K) [C][D]     V [C][M]     A [C][C+p]
//   fp32 side arrays: z [D], column-sum partials, row-sum partials, phi(q).z
// bf16 tiles are unpadded with their 16-byte blocks XOR-swizzled per row (bswz),
// so that both row reads (sixteen rows, one block each) and the transposed reads
// of gfx950 (ds_read_b64_tr_b16: four rows, two blocks each, handed out column
// by column) spread over the LDS banks.  The bf16 MFMA operands that need the
// key index contiguous per lane (phi(K)^T and V^T in the state update, V^T in
// the intra-chunk term, the key sums of phi(K)) come from those transposed reads
// of the natural tiles, so no transposed copy is stored; fp32 MFMA takes one
// element per lane from any layout.
#pragma once

#include <type_traits>

#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

constexpr size_t kMaxLds = 160 * 1024;

template <typename T, int D, int M, int C>
struct Cfg {
    static constexpr bool F32 = std::is_same<T, float>::value;
    static constexpr int RT = C / 16, DT = D / 16, MT = M / 16;
    // Wavefronts per workgroup: one per 16-column m-tile when M = 128 (two per
    // SIMD, half the registers per wavefront), else four.
    static constexpr int NW = MT >= 8 ? 8 : 4;
    static constexpr int THREADS = 64 * NW;
    // Workgroups per CU the register budget is sized for.
    static constexpr int MIN_WG = (NW == 4 && D * M <= 4096) ? 2 : 1;
    static constexpr int MTW = (MT + NW - 1) / NW;  // m-tiles per wavefront
    static constexpr int NA = RT * (RT + 1) / 2;            // lower-triangle tiles of A
    static constexpr int PAD = F32 ? 12 : 8;
    static constexpr int LQ = F32 ? D + PAD : D;  // rows of phi(Q), phi(K) (bf16: swizzled, unpadded)
    static constexpr int LA = C + PAD;            // rows of A
    static constexpr int LV = F32 ? M + PAD : M;  // rows of V (bf16: swizzled, unpadded)
    static constexpr int E = D * M + D; // floats of one state (S then z)
    static constexpr int EP = (E + 63) / 64 * 64;  // exchanged-state slot: whole 256-byte blocks
    static constexpr int NZP = THREADS / D < C ? THREADS / D : C;  // column-sum partial groups
    static constexpr int ZROWS = C / NZP;                            // rows per partial
    static_assert(ZROWS * NZP == C && NZP * D <= THREADS, "column-sum split");
    static constexpr int TPR = THREADS / C < D ? THREADS / C : D;    // threads per row of phi(q).z
    static_assert(TPR <= 64 && (64 % TPR) == 0 && TPR * C <= THREADS, "phi(q).z split");

    // T-element offsets
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + C * LQ;
    static constexpr int oV = oK + C * LQ;
    static constexpr int nV = C * LV;
    static constexpr int oA = oV + nV;
    static constexpr int nT = oA + C * LA;
    static constexpr size_t fbase = ((nT * sizeof(T) + 15) / 16) * 16;
    // float offsets (from fbase)
    static constexpr int fz = 0;
    static constexpr int fzp = fz + D;
    static constexpr int fdenp = fzp + (NZP > 0 ? NZP : 1) * D;
    static constexpr int fqz = fdenp + 4 * RT * C;  // sdenp: [kt][lane group][query]
    static constexpr int nF = fqz + C;
    static constexpr size_t bytes = fbase + nF * sizeof(float);
    static constexpr bool fits = bytes + 64 <= kMaxLds;
};

// ---------------------------------------------------------------------------
// Staging of a C x W tile of a [N][W] head matrix: global -> registers -> LDS.
// An item is one 16-byte vector of one row (rows of W/VEC items).
// Rows at or beyond N are stored as zeros (after phi, so they add nothing).
// ---------------------------------------------------------------------------
// Swizzle of the bf16 tiles: a row of NB 16-byte blocks (NB = W / 8 <= 16) keeps
// its logical block b at position b ^ bswz<NB>(row).  With R = 16 / NB rows in
// one 256-byte window of the LDS banks and a = row / R, bswz = (2a + a / (NB/2))
// mod NB: sixteen consecutive rows put one logical block in sixteen different
// bank groups (row reads of MFMA operands), and four consecutive rows put a pair
// of blocks (2j, 2j+1) in eight different bank groups (transposed reads).
template <int NB>
__device__ __forceinline__ int bswz(int row) {
    static_assert(NB >= 2 && NB <= 16 && (NB & (NB - 1)) == 0, "blocks per row");
    constexpr int R = 16 / NB;
    constexpr int SH = NB == 16 ? 3 : NB == 8 ? 2 : NB == 4 ? 1 : 0;
    const int a = row / R;
    return (2 * a + (a >> SH)) & (NB - 1);
}
// element offset of logical block b (8 elements) of row r in a swizzled tile W wide
template <int W>
__device__ __forceinline__ int boff(int r, int b) {
    return r * W + ((b ^ bswz<W / 8>(r)) << 3);
}
// 8 elements (logical block b) / 4 elements from column c (c % 4 == 0) of row r
template <int W>
__device__ __forceinline__ bf16x8 rd8(const bf16 *tile, int r, int b) {
    return *reinterpret_cast<const bf16x8 *>(tile + boff<W>(r, b));
}
template <int W>
__device__ __forceinline__ bf16x4 rd4(const bf16 *tile, int r, int c) {
    return *reinterpret_cast<const bf16x4 *>(tile + boff<W>(r, c >> 3) + (c & 7));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// Transposed read (ds_read_b64_tr_b16) of a swizzled bf16 tile [keys][W]: within
// each group of 16 lanes, lane j names 4 consecutive elements (row key_j, columns
// col0 + 4 (j % 4) ..), and lane i receives column i % 4 of the rows named by
// lanes i / 4 + 4k, k = 0..3.  With key_j = kb + j / 4 lane l16 receives
// tile[kb .. kb + 3][col0 + l16]: four keys of one column, the layout of a
// 4-deep slice of an MFMA operand whose contraction index is the key.
template <int W>
__device__ __forceinline__ bf16x4 tr4(const bf16 *tile, int kb, int col0, int l16) {
    const int key = kb + (l16 >> 2);
    const int b = (col0 >> 3) + ((l16 & 3) >> 1);
    const bf16 *p = tile + key * W + ((b ^ bswz<W / 8>(key)) << 3) + 4 * (l16 & 1);
    const s16x4 v =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(const_cast<bf16 *>(p)));
    return __builtin_bit_cast(bf16x4, v);
}
// the 32-deep operand slice of lane (g, l16): keys kb + 8g .. kb + 8g + 7 of column col0 + l16
template <int W>
__device__ __forceinline__ bf16x8 tr8(const bf16 *tile, int kb, int col0, int g, int l16) {
    const bf16x4 lo = tr4<W>(tile, kb + 8 * g, col0, l16);
    const bf16x4 hi = tr4<W>(tile, kb + 8 * g + 4, col0, l16);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <typename T, int C, int W, int NT>
struct Stage {
    static constexpr bool F32 = std::is_same<T, float>::value;
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr int NV = W / VEC;
    static constexpr int RPI = 1;  // rows per item
    static constexpr int ITEMS = (C / RPI) * NV;
    static constexpr int PER = (ITEMS + NT - 1) / NT;
    uint4 r[PER][RPI];

    template <bool NTL = false>
    __device__ __forceinline__ void load(const T *__restrict__ head, int row0, int N, int tid) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int item = tid + p * NT;
            if (ITEMS % NT == 0 || item < ITEMS) {
                const int rq = item / NV, cv = item % NV;
#pragma unroll
                for (int i = 0; i < RPI; ++i) {
                    // rows past the end re-read the last row (no branch); the stores zero them.
                    // NTL (the two-phase kernel's passes): nontemporal, each row streams through
                    // once per pass and the second pass starts long after the first has left the
                    // caches (417 -> 400 us on a 16 x 65536-row bf16 head set); the one-pass
                    // kernel keeps cached loads (nontemporal ones cost its 16-token decode 10 %).
                    const int grow = min(row0 + rq * RPI + i, N - 1);
                    if constexpr (NTL)
                        r[p][i] = __builtin_bit_cast(
                            uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(head + (size_t)grow * W + cv * VEC)));
                    else
                        r[p][i] = *reinterpret_cast<const uint4 *>(head + (size_t)grow * W + cv * VEC);
                }
            }
        }
    }

    // natural layout dst[row][col], optionally through phi; SWZ (bf16 tiles W wide):
    // blocks swizzled per row (bswz).  Rows at or past N (only in the last chunk)
    // are zeroed; full chunks take a branch-free path.
    template <bool PHI, bool SWZ = false>
    __device__ __forceinline__ void store_natural(T *dst, int ld, int row0, int N, int tid) const {
        if (row0 + C <= N)
            store_natural_impl<PHI, false, SWZ>(dst, ld, row0, N, tid);
        else
            store_natural_impl<PHI, true, SWZ>(dst, ld, row0, N, tid);
    }
    // fp32 copy dst[row][col] of the tile (natural layout, no phi); rows at or
    // past N are zeroed.  For fp32 tiles this is store_natural<false>.
    __device__ __forceinline__ void store_natural_f32(float *dst, int ld, int row0, int N, int tid) const {
        if constexpr (F32) {
            store_natural<false>(dst, ld, row0, N, tid);
        } else {
#pragma unroll
            for (int p = 0; p < PER; ++p) {
                const int item = tid + p * NT;
                if (ITEMS % NT == 0 || item < ITEMS) {
                    const int rq = item / NV, cv = item % NV;
#pragma unroll
                    for (int i = 0; i < RPI; ++i) {
                        const int row = rq * RPI + i;
                        const float keep = row0 + row < N ? 1.0f : 0.0f;
                        const bf16x8 x = __builtin_bit_cast(bf16x8, r[p][i]);
                        f32x4 lo, hi;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            lo[j] = (float)x[j] * keep;
                            hi[j] = (float)x[4 + j] * keep;
                        }
                        *reinterpret_cast<f32x4 *>(dst + row * ld + cv * 8) = lo;
                        *reinterpret_cast<f32x4 *>(dst + row * ld + cv * 8 + 4) = hi;
                    }
                }
            }
        }
    }
    template <bool PHI, bool TAIL, bool SWZ = false>
    __device__ __forceinline__ void store_natural_impl(T *dst, int ld, int row0, int N, int tid) const {
        static_assert(!SWZ || !F32, "swizzled tiles are bf16");
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int item = tid + p * NT;
            if (ITEMS % NT == 0 || item < ITEMS) {
                const int rq = item / NV, cv = item % NV;
#pragma unroll
                for (int i = 0; i < RPI; ++i) {
                    const int row = rq * RPI + i;
                    const float keep = (!TAIL || row0 + row < N) ? 1.0f : 0.0f;
                    if constexpr (F32) {
                        f32x4 x = __builtin_bit_cast(f32x4, r[p][i]);
                        f32x4 y;
#pragma unroll
                        for (int j = 0; j < 4; ++j) y[j] = (PHI ? phi(x[j]) : x[j]) * keep;
                        *reinterpret_cast<f32x4 *>(dst + row * ld + cv * 4) = y;
                    } else {
                        bf16x8 x = __builtin_bit_cast(bf16x8, r[p][i]);
                        bf16x8 y;
                        if constexpr (!PHI && !TAIL) {
                            y = x;  // a plain copy
                        } else {
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                const float f = (float)x[j];
                                y[j] = (bf16)((PHI ? phi(f) : f) * keep);
                            }
                        }
                        const int blk = SWZ ? (cv ^ bswz<NV>(row)) : cv;
                        *reinterpret_cast<bf16x8 *>(dst + row * ld + blk * 8) = y;
                    }
                }
            }
        }
    }

};


// ---------------------------------------------------------------------------
// Workspace of the fused kernel (fp32 words):
//   header (64 words): [1] finished-head counter, [2] epoch,
//                      [3] error flag (look-back gave up)
//   flags  [BH][G] (uint32, padded to 64 words): epoch << 2 | 1 aggregate ready,
//                                                epoch << 2 | 2 inclusive ready
//   aggregate states [BH][G][EP], inclusive states [BH][G][EP] (EP: E padded to
//   whole 256-byte blocks; the slot layout is the lane order of the register
//   tiles, see Engine::slot_store)
// The header and flags must be zero before the first call with a given plan;
// the last workgroup of every call resets the counters and advances the
// epoch, which makes all flags of the call stale.
// ---------------------------------------------------------------------------
struct FusedWs {
    unsigned *hdr;
    unsigned *flags;
    float *agg;
    float *incl;
    __device__ FusedWs(void *ws, long BH, int G, int E) {
        hdr = static_cast<unsigned *>(ws);
        flags = hdr + kWsHeaderWords;
        agg = reinterpret_cast<float *>(flags + fused_flag_words((long)BH * G));
        incl = agg + (size_t)BH * G * fused_slot_floats(E);
    }
};

// ---------------------------------------------------------------------------
// The per-chunk engine shared by the kernels.
// ---------------------------------------------------------------------------
// PHI: apply the feature map phi while staging Q and K (false: the inputs already
// hold features, e.g. random features computed by the feature-map kernel).
template <typename T, int D, int M, int C, bool PHI = true>
struct Engine {
    using G = Cfg<T, D, M, C>;
    static constexpr int DT = G::DT, MTW = G::MTW, RT = G::RT;
    T *sQ, *sK, *sV, *sA;
    float *sz, *szp, *sdenp, *sqz;
    int tid, lane, w, g, l16;

    __device__ __forceinline__ explicit Engine(unsigned char *smem) {
        T *t = reinterpret_cast<T *>(smem);
        sQ = t + G::oQ;
        sK = t + G::oK;
        sV = t + G::oV;
        sA = t + G::oA;
        float *f = reinterpret_cast<float *>(smem + G::fbase);
        sz = f + G::fz;
        szp = f + G::fzp;
        sdenp = f + G::fdenp;
        sqz = f + G::fqz;
        tid = threadIdx.x;
        lane = tid & 63;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile choices become scalar branches
        g = lane >> 4;
        l16 = lane & 15;
    }

    __device__ __forceinline__ bool owns(int i) const { return G::MT % G::NW == 0 || w + G::NW * i < G::MT; }

    // z[tid] of the running sums for the phi(q) . z products (thread tid < D): fp32,
    // or rounded to bf16 (stored packed in the first half of sz) for the bf16 engine
    __device__ __forceinline__ void set_z(float z) const {
        if constexpr (G::F32)
            sz[tid] = z;
        else
            reinterpret_cast<bf16 *>(sz)[tid] = (bf16)z;
    }
    __device__ __forceinline__ int mtile(int i) const { return w + G::NW * i; }

    // The upper triangle of A is never written by a_tiles; zero it (all of A) once.
    __device__ __forceinline__ void clear_a() const {
        for (int e = tid; e < C * G::LA; e += G::THREADS) sA[e] = from_f32<T>(0.0f);
    }

    __device__ __forceinline__ void store_q(const Stage<T, C, D, Cfg<T, D, M, C>::THREADS> &st, int row0, int N) const {
        st.template store_natural<PHI, !G::F32>(sQ, G::LQ, row0, N, tid);
    }
    __device__ __forceinline__ void store_kv(const Stage<T, C, D, Cfg<T, D, M, C>::THREADS> &stK, const Stage<T, C, M, Cfg<T, D, M, C>::THREADS> &stV, int row0,
                                             int N) const {
        if constexpr (G::F32) {
            stK.template store_natural<PHI>(sK, G::LQ, row0, N, tid);
            stV.template store_natural<false>(sV, G::LV, row0, N, tid);
        } else {
            stK.template store_natural<PHI, true>(sK, G::LQ, row0, N, tid);
            stV.template store_natural<false, true>(sV, G::LV, row0, N, tid);
        }
    }

    // Column sums of phi(K_c).  fp32: partial sums over ZROWS rows into szp[q][d].
    // bf16: phi(K_c)^T 1 on MFMA (the key-contiguous operand from transposed reads,
    // a B operand of ones), wavefront w summing the d-tiles w, w + NW, ...; the
    // result row d of the tile lands in szp[d].
    static constexpr int ZP = G::F32 ? G::NZP : 1;  // partials per column
    __device__ __forceinline__ void z_partials() const {
        if constexpr (G::F32) {
            const int q = tid / D, d = tid % D;
            if (G::NZP * D == G::THREADS || q < G::NZP) {
                float s = 0.0f;
#pragma unroll
                for (int r = 0; r < G::ZROWS; ++r) s += to_f32(sK[(q * G::ZROWS + r) * G::LQ + d]);
                szp[q * D + d] = s;
            }
        } else {
            const bf16 one = (bf16)1.0f;
            for (int dt = w; dt < DT; dt += G::NW) {
                f32x4 acc = zero4();
                if constexpr (C % 32 == 0) {
                    const bf16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
                    for (int ks = 0; ks < C / 32; ++ks) acc = mma_bf16_k32(tr8<D>(sK, ks * 32, dt * 16, g, l16), ones, acc);
                } else {
                    const bf16x4 ones = {one, one, one, one};
                    acc = mma_bf16_k16(tr4<D>(sK, 4 * g, dt * 16, l16), ones, acc);
                }
                if (l16 == 0) *reinterpret_cast<f32x4 *>(szp + dt * 16 + 4 * g) = acc;
            }
        }
    }
    __device__ __forceinline__ float z_delta() const {  // thread tid < D, after a barrier
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < ZP; ++q) s += szp[q * D + tid];
        return s;
    }

    // S[:, own m-tiles] += phi(K_c)^T V_c.  acc[dt][i][r] = S[dt*16 + 4g + r][mt_i*16 + l16].
    __device__ __forceinline__ void state_update(f32x4 (&acc)[DT][MTW]) const {
        if constexpr (G::F32) {
#pragma unroll 4
            for (int ks = 0; ks < C / 4; ++ks) {
                const int key = 4 * ks + g;
                float bv[MTW];
#pragma unroll
                for (int i = 0; i < MTW; ++i) bv[i] = owns(i) ? sV[key * G::LV + mtile(i) * 16 + l16] : 0.0f;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const float a = sK[key * G::LQ + dt * 16 + l16];
#pragma unroll
                    for (int i = 0; i < MTW; ++i)
                        if (owns(i)) acc[dt][i] = mma_f32(a, bv[i], acc[dt][i]);
                }
            }
        } else {
            // A = phi(K)^T (rows d, keys), B = V (keys, columns m): both from transposed reads
#pragma unroll
            for (int i = 0; i < MTW; ++i) {
                if (!owns(i)) continue;
                const int mc = mtile(i) * 16;
                if constexpr (C % 32 == 0) {
                    bf16x8 bv[C / 32];
#pragma unroll
                    for (int ks = 0; ks < C / 32; ++ks) bv[ks] = tr8<M>(sV, ks * 32, mc, g, l16);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                        for (int ks = 0; ks < C / 32; ++ks)
                            acc[dt][i] = mma_bf16_k32(tr8<D>(sK, ks * 32, dt * 16, g, l16), bv[ks], acc[dt][i]);
                } else {
                    const bf16x4 bv = tr4<M>(sV, 4 * g, mc, l16);
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        acc[dt][i] = mma_bf16_k16(tr4<D>(sK, 4 * g, dt * 16, l16), bv, acc[dt][i]);
                }
            }
        }
    }

    // Lower-triangle tiles of A (tile t = w, w+NW, ... in row-major order of (rt, kt<=rt)),
    // rounded to T, into sA[query][key]; each lane group's share of their row sums
    // into sdenp[kt][g][query] (summed by row_den after the next barrier, instead of
    // two cross-lane exchanges here on the chunk's critical path).  All of
    // a wavefront's tile products are issued before any epilogue, so their latencies
    // overlap.
    static __device__ __forceinline__ int tile_row(int t) {
        int rt = 0;
        while ((rt + 1) * (rt + 2) / 2 <= t) ++rt;
        return rt;
    }
    __device__ __forceinline__ void a_tiles() const {
        constexpr int NTW = (G::NA + G::NW - 1) / G::NW;  // tiles per wavefront (at most)
        f32x4 acc[NTW];
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
            const int t = w + G::NW * k;
            acc[k] = zero4();
            if (G::NA % G::NW == 0 || t < G::NA) {
                const int rt = tile_row(t), kt = t - rt * (rt + 1) / 2;
                if constexpr (G::F32) {
                    const T *krow = sK + (kt * 16 + l16) * G::LQ;
                    const T *qrow = sQ + (rt * 16 + l16) * G::LQ;
                    // contraction index d = g*(D/4) + j: each lane reads a contiguous quarter of the row
#pragma unroll
                    for (int j4 = 0; j4 < D / 16; ++j4) {
                        const f32x4 av = *reinterpret_cast<const f32x4 *>(krow + g * (D / 4) + 4 * j4);
                        const f32x4 bv = *reinterpret_cast<const f32x4 *>(qrow + g * (D / 4) + 4 * j4);
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[k] = mma_f32(av[j], bv[j], acc[k]);
                    }
                } else {
                    // contraction slots of lane (g, l16): logical block 4 ks + g of the rows
                    const int kr = kt * 16 + l16, qr = rt * 16 + l16;
                    if constexpr (D % 32 == 0) {
#pragma unroll
                        for (int ks = 0; ks < D / 32; ++ks)
                            acc[k] = mma_bf16_k32(rd8<D>(sK, kr, 4 * ks + g), rd8<D>(sQ, qr, 4 * ks + g), acc[k]);
                    } else {
                        static_assert(D == 16, "bf16 widths are 16, 32, 64 or 128");
                        acc[k] = mma_bf16_k16(rd4<D>(sK, kr, 4 * g), rd4<D>(sQ, qr, 4 * g), acc[k]);
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
            const int t = w + G::NW * k;
            if (G::NA % G::NW == 0 || t < G::NA) {
                const int rt = tile_row(t), kt = t - rt * (rt + 1) / 2;
                f32x4 a = acc[k];
                // a[r] = A[query = rt*16 + l16][key = kt*16 + 4g + r]
                if (kt == rt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * g + r > l16) a[r] = 0.0f;
                }
                float rs = 0.0f;
                T *arow = sA + (rt * 16 + l16) * G::LA + kt * 16 + 4 * g;
                if constexpr (G::F32) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) rs += a[r];
                    *reinterpret_cast<f32x4 *>(arow) = a;
                } else {
                    // the row sum of the rounded values (those the intra-chunk product uses),
                    // by two dot2 instructions against ones
                    const bf16x4 v = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]};
                    const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
                    rs = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[0], v[1]}, one2, 0.0f, false);
                    rs = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2], v[3]}, one2, rs, false);
                    *reinterpret_cast<bf16x4 *>(arow) = v;
                }
                sdenp[(kt * 4 + g) * C + rt * 16 + l16] = rs;
            }
        }
    }

    // phi(q_i) . z for every row i of the chunk -> dst[i] (default sqz)
    __device__ __forceinline__ void qz_rows() const { qz_rows_to(sqz); }
    __device__ __forceinline__ void qz_rows_to(float *dst) const {
        constexpr int TPR = G::TPR;  // threads per row, consecutive lanes
        constexpr int EPT = D / TPR;  // elements per thread, contiguous
        constexpr int VW = 16 / (int)sizeof(T);
        const int i = tid / TPR, p = tid % TPR;
        if (G::TPR * C < G::THREADS && i >= C) return;  // whole wavefronts beyond the rows
        const T *qr = sQ + i * G::LQ + p * EPT;  // fp32 rows are plain
        const float *zr = sz + p * EPT;
        float s = 0.0f;
        if constexpr (EPT % VW == 0) {
            // 16-byte reads of the phi(q) row and of z
#pragma unroll
            for (int v = 0; v < EPT / VW; ++v) {
                if constexpr (G::F32) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(qr + 4 * v);
                    const f32x4 b = *reinterpret_cast<const f32x4 *>(zr + 4 * v);
#pragma unroll
                    for (int j = 0; j < 4; ++j) s += a[j] * b[j];
                } else {
                    // packed bf16 pairs of phi(q) and z: two products per dot2 instruction
                    const bf16x8 a = rd8<D>(sQ, i, (p * EPT) / 8 + v);
                    const bf16x8 b = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const bf16 *>(sz) + p * EPT + 8 * v);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        s = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[2 * j], a[2 * j + 1]}, bf16x2{b[2 * j], b[2 * j + 1]}, s,
                                                            false);
                }
            }
        } else if constexpr (G::F32) {
#pragma unroll
            for (int j = 0; j < EPT; ++j) s += qr[j] * zr[j];
        } else {
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                const int col = p * EPT + j;
                s += to_f32(sQ[boff<D>(i, col >> 3) + (col & 7)]) * (float)reinterpret_cast<const bf16 *>(sz)[col];
            }
        }
        s = row_group_sum<(TPR < 16 ? TPR : 16)>(s);
        if constexpr (TPR >= 32) s += __shfl_xor(s, 16, 64);
        if constexpr (TPR >= 64) s += __shfl_xor(s, 32, 64);
        if (p == 0) dst[i] = s;
    }

    // den for row `lane` (lanes >= C return 1); needs sdenp and sqz (after a barrier)
    template <bool CAUSAL>
    __device__ __forceinline__ float row_den() const {
        if (lane >= C) return 1.0f;
        const int rt = lane / 16;
        float den = sqz[lane];
        if constexpr (CAUSAL) {
#pragma unroll
            for (int kt = 0; kt < RT; ++kt)
                if (kt <= rt) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) den += sdenp[(kt * 4 + q) * C + lane];
                }
        }
        return den;
    }
    template <bool CAUSAL>
    __device__ __forceinline__ float row_inv() const {
        return 1.0f / row_den<CAUSAL>();
    }

    // Output tiles of the chunk for the own m-tiles.  Each MFMA takes the V / S side
    // as its A operand and the A / phi(Q) side as its B operand, so a result tile is
    // out^T: lane (g, l16) holds out[query rt*16 + l16][m*16 + 4g .. +3], four
    // consecutive columns, stored with one 16-byte write.
    //   intra():   o += (A V_c)^T           (needs sA, V; not the earlier state)
    //   readout(): o += (phi(Q_c) S)^T, then o * inv -> out   (S from registers)
    __device__ __forceinline__ void intra(f32x4 (&o)[RT][MTW]) const {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int qrow = rt * 16 + l16;
            if constexpr (G::F32) {
                const int nsteps = 4 * (rt + 1);  // keys per lane group: g*nsteps .. (g+1)*nsteps-1
                const float *arow = sA + qrow * G::LA + g * nsteps;
#pragma unroll
                for (int j4 = 0; j4 < rt + 1; ++j4) {
                    const f32x4 av = *reinterpret_cast<const f32x4 *>(arow + 4 * j4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = g * nsteps + 4 * j4 + j;
#pragma unroll
                        for (int i = 0; i < MTW; ++i)
                            if (owns(i)) o[rt][i] = mma_f32(sV[key * G::LV + mtile(i) * 16 + l16], av[j], o[rt][i]);
                    }
                }
            } else if constexpr (RT == 1) {
                const bf16x4 bv = *reinterpret_cast<const bf16x4 *>(sA + qrow * G::LA + 4 * g);
#pragma unroll
                for (int i = 0; i < MTW; ++i) {
                    if (!owns(i)) continue;
                    o[rt][i] = mma_bf16_k16(tr4<M>(sV, 4 * g, mtile(i) * 16, l16), bv, o[rt][i]);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < (rt + 2) / 2; ++kk) {
                    const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(sA + qrow * G::LA + kk * 32 + 8 * g);
#pragma unroll
                    for (int i = 0; i < MTW; ++i) {
                        if (!owns(i)) continue;
                        o[rt][i] = mma_bf16_k32(tr8<M>(sV, kk * 32, mtile(i) * 16, g, l16), bv, o[rt][i]);
                    }
                }
            }
        }
    }

    // o += (phi(Q_c) S)^T for the chunk's rows of sQ, S from registers
    __device__ __forceinline__ void readout_mma(f32x4 (&o)[RT][MTW], const f32x4 (&S)[DT][MTW]) const {
        if constexpr (G::F32) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int qrow = rt * 16 + l16;
                // contraction slot of lane (g, l16) at step (dt, r) is d = dt*16 + 4g + r
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const f32x4 qv = *reinterpret_cast<const f32x4 *>(sQ + qrow * G::LQ + dt * 16 + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int i = 0; i < MTW; ++i)
                            if (owns(i)) o[rt][i] = mma_f32(S[dt][i][r], qv[r], o[rt][i]);
                }
            }
        } else if constexpr (DT == 1) {
            bf16x4 sb[MTW];
#pragma unroll
            for (int i = 0; i < MTW; ++i)
                sb[i] = bf16x4{(bf16)S[0][i][0], (bf16)S[0][i][1], (bf16)S[0][i][2], (bf16)S[0][i][3]};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int qrow = rt * 16 + l16;
                const bf16x4 qv = rd4<D>(sQ, qrow, 4 * g);
#pragma unroll
                for (int i = 0; i < MTW; ++i)
                    if (owns(i)) o[rt][i] = mma_bf16_k16(sb[i], qv, o[rt][i]);
            }
        } else {
            // the bf16 copy of the state is made once per call, not per row tile
            bf16x8 sv[DT / 2][MTW];
#pragma unroll
            for (int p = 0; p < DT / 2; ++p)
#pragma unroll
                for (int i = 0; i < MTW; ++i) {
                    const f32x4 s0 = S[2 * p][i], s1 = S[2 * p + 1][i];
                    sv[p][i] = bf16x8{(bf16)s0[0], (bf16)s0[1], (bf16)s0[2], (bf16)s0[3],
                                      (bf16)s1[0], (bf16)s1[1], (bf16)s1[2], (bf16)s1[3]};
                }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int qrow = rt * 16 + l16;
#pragma unroll
                for (int p = 0; p < DT / 2; ++p) {
                    const bf16x4 q0 = rd4<D>(sQ, qrow, (2 * p) * 16 + 4 * g);
                    const bf16x4 q1 = rd4<D>(sQ, qrow, (2 * p + 1) * 16 + 4 * g);
                    const bf16x8 qv = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
#pragma unroll
                    for (int i = 0; i < MTW; ++i)
                        if (owns(i)) o[rt][i] = mma_bf16_k32(sv[p][i], qv, o[rt][i]);
                }
            }
        }
    }

    // out[row0 + rows] = o * (1 / den) of the row (inv: lane r holds row r's factor).
    // OT = float: 16-byte stores; OT = bf16: rounded to nearest even, 8-byte stores.
    template <typename OT>
    __device__ __forceinline__ void store_rows(const f32x4 (&o)[RT][MTW], float inv, OT *__restrict__ Oh, int row0,
                                               int N, bool poison) const {
        const bool full = row0 + C <= N;  // uniform: no per-row bounds checks needed
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int qrow = rt * 16 + l16;
            const float inv_q = __shfl(inv, qrow, 64);
            const int grow = row0 + qrow;
            if (full || grow < N) {
#pragma unroll
                for (int i = 0; i < MTW; ++i) {
                    if (!owns(i)) continue;
                    f32x4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = poison ? __builtin_nanf("") : o[rt][i][r] * inv_q;
                    OT *dst = Oh + (size_t)grow * M + mtile(i) * 16 + 4 * g;
                    if constexpr (std::is_same<OT, float>::value) {
                        *reinterpret_cast<f32x4 *>(dst) = v;
                    } else {
                        *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
                    }
                }
            }
        }
    }

    template <typename OT>
    __device__ __forceinline__ void readout(f32x4 (&o)[RT][MTW], const f32x4 (&S)[DT][MTW], float inv,
                                            OT *__restrict__ Oh, int row0, int N, bool poison) const {
        readout_mma(o, S);
        store_rows(o, inv, Oh, row0, N, poison);
    }

    __device__ __forceinline__ static void zero_out(f32x4 (&o)[RT][MTW]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < MTW; ++i) o[rt][i] = zero4();
    }

    // ---- state slots ([D][M] row major, then z[D]) <-> register layout ----
    __device__ __forceinline__ void state_store(const f32x4 (&acc)[DT][MTW], float z, float *Sd, float *zd) const {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < MTW; ++i) {
                if (!owns(i)) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) Sd[(dt * 16 + 4 * g + r) * M + mtile(i) * 16 + l16] = acc[dt][i][r];
            }
        if (tid < D) zd[tid] = z;
    }
    __device__ __forceinline__ void state_store(const f32x4 (&acc)[DT][MTW], float z, float *slot) const {
        state_store(acc, z, slot, slot + D * M);
    }
    __device__ __forceinline__ void state_add(f32x4 (&acc)[DT][MTW], float &z, const float *Sd,
                                              const float *zd) const {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < MTW; ++i) {
                if (!owns(i)) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[dt][i][r] += Sd[(dt * 16 + 4 * g + r) * M + mtile(i) * 16 + l16];
            }
        if (tid < D) z += zd[tid];
    }
    __device__ __forceinline__ void state_add(f32x4 (&acc)[DT][MTW], float &z, const float *slot) const {
        state_add(acc, z, slot, slot + D * M);
    }
    // ---- states exchanged between workgroups (fused and one-pass kernels) ----
    // Slot layout (private to these kernels): the register tiles in lane order,
    // tile (dt, mt) at floats ((dt*MT + mt)*64 + lane)*4 .. +3, then z[D] at D*M;
    // slots are padded to whole 256-byte blocks so that no cache line is shared
    // between slots.  Writers store write-through at agent scope (buffer stores
    // with sc1); a flag is raised only after the stores complete.  Readers load
    // a slot only after its flag, with plain cacheable loads: each slot is
    // written once per call and never read before its flag, so no stale copy of
    // it can be cached (caches are invalidated at kernel start).
    __device__ __forceinline__ int xoff(int dt, int i) const { return ((dt * G::MT + mtile(i)) * 64 + lane) * 4; }
    __device__ __forceinline__ void slot_store(const f32x4 (&acc)[DT][MTW], float z, float *slot) const {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(slot, (short)0, G::EP * 4, 0x00020000);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < MTW; ++i) {
                if (!owns(i)) continue;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[dt][i]), rs, xoff(dt, i) * 4, 0,
                                                       kCachePolicyAgent);
            }
        if (tid < D) __hip_atomic_store(slot + D * M + tid, z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // pre += *first + agg[j0] + ... + agg[j1-1] (slots of EP floats), loads issued NB
    // slots at a time so that their latencies overlap; fixed summation order.
    __device__ __forceinline__ void state_add_slots(f32x4 (&acc)[DT][MTW], float &z, const float *first,
                                                    const float *agg, int j0, int j1) const {
        constexpr int PER = DT * MTW;  // 16-byte loads per slot and lane
        constexpr int NB = PER <= 4 ? 4 : (PER <= 8 ? 2 : 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < MTW; ++i)
                if (owns(i)) acc[dt][i] += *reinterpret_cast<const f32x4 *>(first + xoff(dt, i));
        if (tid < D) z += first[D * M + tid];
        for (int jb = j0; jb < j1; jb += NB) {
            f32x4 t[NB][DT][MTW];
            float tz[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const float *slot = agg + (size_t)(jb + k < j1 ? jb + k : jb) * G::EP;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int i = 0; i < MTW; ++i)
                        t[k][dt][i] = owns(i) ? *reinterpret_cast<const f32x4 *>(slot + xoff(dt, i)) : zero4();
                tz[k] = tid < D ? slot[D * M + tid] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                if (jb + k >= j1) break;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int i = 0; i < MTW; ++i) acc[dt][i] += t[k][dt][i];
                z += tz[k];
            }
        }
    }

    // Publish: wait until this wave's coherent stores are complete, then let one
    // thread raise the flag once every wave of the workgroup has done so.
    __device__ __forceinline__ void publish_flag(unsigned *flag, unsigned value) const {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0) __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    __device__ __forceinline__ static void zero_state(f32x4 (&acc)[DT][MTW]) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < MTW; ++i) acc[dt][i] = zero4();
    }
};

// ---------------------------------------------------------------------------
// Phase A: sum the state over chunks [c0, c1) into acc / z (thread tid < D owns z[tid]).
// Leaves the last chunk's phi(K), V in LDS.  Global loads run two chunks ahead.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
template <int DI, int F, int C>
struct FeatLds {
    static constexpr int LX = DI + 4;           // LDS row of a raw tile
    static constexpr int WROWS = (F + 15) / 16 * 16;
    static constexpr int nRaw = 2 * C * LX;     // raw q, raw k
    static constexpr int nW = WROWS * LX;
    static constexpr size_t bytes = (size_t)(nRaw + nW) * 4;
    static_assert(DI % 16 == 0, "16-deep contraction blocks");
};

// One (tensor, 16-row tile, 16-projection tile) job of the projection: lane
// (g, l16) ends with projections 4g .. 4g+3 of row l16 (W rows as the MFMA A
// operand, x rows as B; within each 16-deep block lane g contracts over
// k = 16 kb + 4 g + kk for both).
template <int DI, int F, int C>
__device__ __forceinline__ void feature_job(const float *raw, const float *sw, float *dst, int ld, int rt, int pt,
                                            int P, int kind, bool norm, int row0, int N, int lane) {
    using FL = FeatLds<DI, F, C>;
    const int g = lane >> 4, l16 = lane & 15;
    const float *xr = raw + (rt * 16 + l16) * FL::LX + 4 * g;
    const float *wr = sw + (pt * 16 + l16) * FL::LX + 4 * g;
    f32x4 acc = zero4();
    float sq = 0.0f;
#pragma unroll
    for (int kb = 0; kb < DI / 16; ++kb) {
        const f32x4 b = *reinterpret_cast<const f32x4 *>(xr + 16 * kb);
        const f32x4 a = *reinterpret_cast<const f32x4 *>(wr + 16 * kb);
        sq += b[0] * b[0] + b[1] * b[1] + b[2] * b[2] + b[3] * b[3];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mma_f32(a[kk], b[kk], acc);
    }
    sq += __shfl_xor(sq, 16, 64);  // the four lanes g of row l16 hold a quarter each
    sq += __shfl_xor(sq, 32, 64);
    float scale = 1.0f;
    if (norm && sq > 0.0f) {
        scale = 1.0f / sqrtf(sq);
        sq = sq * scale * scale;
    }
    const int row = rt * 16 + l16, f0 = pt * 16 + 4 * g;
    if (f0 >= P) return;
    const bool pad = row0 + row >= N;
    float *o = dst + row * ld;
    if (kind == 1) {
        const float inv = 1.0f / sqrtf((float)F);
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = pad ? 0.0f : __expf(acc[r] * scale - 0.5f * sq) * inv;
        *reinterpret_cast<f32x4 *>(o + f0) = v;
    } else {
        const float c = __expf(0.5f * sq) / sqrtf((float)P);
        f32x4 vs, vc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float sn, cs;
            sincosf(acc[r] * scale, &sn, &cs);
            vs[r] = pad ? 0.0f : c * sn;
            vc[r] = pad ? 0.0f : c * cs;
        }
        *reinterpret_cast<f32x4 *>(o + f0) = vs;
        *reinterpret_cast<f32x4 *>(o + P + f0) = vc;
    }
}

// DK: width of the K rows in memory; TI: their element type (the engine's T
// unless raw rows are mapped to fp32 features while staged)
template <typename T, int D, int M, int C, int DK = D, typename TI = T>
struct KVBuf {
    Stage<TI, C, DK, Cfg<T, D, M, C>::THREADS> k;
    Stage<TI, C, M, Cfg<T, D, M, C>::THREADS> v;
    template <bool NTL = false>
    __device__ __forceinline__ void load(const TI *Kh, const TI *Vh, int c, int N, int tid) {
        k.template load<NTL>(Kh, c * C, N, tid);
        v.template load<NTL>(Vh, c * C, N, tid);
    }
};

// How a chunk's rows reach the engine's tiles: through phi (the elu map), or,
// with DI > 0, as raw rows DI wide (element type TI) that are mapped in fp32 to
// the random features of W (fkind, fnorm) once they are in LDS; the engine then
// works on D = F features.  Raw rows go to their own LDS tiles (store_*), and
// map() forms the features after the barrier that follows those stores.
template <typename T, int D, int M, int C, bool PHI, int DI = 0, typename TI = T>
struct ChunkStager {
    static constexpr bool FEAT = DI > 0;
    static constexpr int DQ = FEAT ? DI : D;  // width of the Q, K rows in memory
    using Gc = Cfg<T, D, M, C>;
    using En = Engine<T, D, M, C, PHI>;
    using FL = FeatLds<FEAT ? DI : 16, D, C>;
    using QStage = Stage<TI, C, DQ, Gc::THREADS>;
    static_assert(!FEAT || (std::is_same<T, float>::value && !PHI), "random features: fp32 engine, no elu map");
    static_assert(FEAT || std::is_same<TI, T>::value, "raw rows of another type only with random features");
    float *sRawQ = nullptr, *sRawK = nullptr, *sW = nullptr;
    int P = D, fkind = 0;
    bool fnorm = false;

    // FEAT: W ([P][DI], P = F or F/2) into LDS once per workgroup, rows past P zero
    __device__ __forceinline__ void init(float *sfeat, const float *__restrict__ W, int kind, int norm, int tid) {
        if constexpr (FEAT) {
            sRawQ = sfeat;
            sRawK = sfeat + C * FL::LX;
            sW = sfeat + FL::nRaw;
            fkind = kind;
            fnorm = norm != 0;
            P = kind == 2 ? D / 2 : D;
            for (int x = tid; x < FL::WROWS * (DI / 4); x += Gc::THREADS) {
                const int f = x / (DI / 4), c4 = (x % (DI / 4)) * 4;
                f32x4 v = zero4();
                if (f < P) v = *reinterpret_cast<const f32x4 *>(W + (size_t)f * DI + c4);
                *reinterpret_cast<f32x4 *>(sW + f * FL::LX + c4) = v;
            }
        }
    }
    __device__ __forceinline__ void store_q(const En &e, const QStage &q, int row0, int N) const {
        if constexpr (FEAT)
            q.store_natural_f32(sRawQ, FL::LX, row0, N, e.tid);
        else
            e.store_q(q, row0, N);
    }
    __device__ __forceinline__ void store_kv(const En &e, const KVBuf<T, D, M, C, DQ, TI> &b, int row0, int N) const {
        if constexpr (FEAT) {
            b.k.store_natural_f32(sRawK, FL::LX, row0, N, e.tid);
            b.v.store_natural_f32(e.sV, Gc::LV, row0, N, e.tid);
        } else {
            e.store_kv(b.k, b.v, row0, N);
        }
    }
    // FEAT: the features of the staged q and/or k rows into e.sQ / e.sK (rows at
    // or past N zero), then a barrier; nothing otherwise
    __device__ __forceinline__ void map(const En &e, bool q, bool k, int row0, int N) const {
        if constexpr (FEAT) {
            const int PT = (P + 15) / 16, per = Gc::RT * PT;
            const int j1 = (k ? 2 : 1) * per;
            for (int jb = e.w + (q ? 0 : per); jb < j1; jb += Gc::NW) {
                const int t = jb / per, rt = (jb % per) / PT, pt = jb % PT;
                feature_job<DI, D, C>(t == 0 ? sRawQ : sRawK, sW, t == 0 ? e.sQ : e.sK, Gc::LQ, rt, pt, P, fkind,
                                      fnorm, row0, N, e.lane);
            }
            __syncthreads();
        }
    }
};


template <typename T, int D, int M, int C, bool PHI, int DI = 0, typename TI = T>
__device__ __forceinline__ void phase_a(const Engine<T, D, M, C, PHI> &e, const TI *__restrict__ Kh,
                                        const TI *__restrict__ Vh, int N, int c0, int c1,
                                        f32x4 (&acc)[Cfg<T, D, M, C>::DT][Cfg<T, D, M, C>::MTW], float &z,
                                        const ChunkStager<T, D, M, C, PHI, DI, TI> &st = {}) {
    // Two chunks of loads in flight (two register buffers, the loop unrolled by
    // two): a phase-A chunk has little arithmetic, so one chunk of work does not
    // cover a load's latency.  Every load is issued unconditionally (index clamped
    // to the last chunk; a clamped reload is an L2 hit) so that the compiler's
    // wait counts stay exact; only the arithmetic of the odd last chunk is skipped.
    using KV = KVBuf<T, D, M, C, ChunkStager<T, D, M, C, PHI, DI, TI>::DQ, TI>;
    KV b0, b1;
    b0.template load<true>(Kh, Vh, c0, N, e.tid);
    b1.template load<true>(Kh, Vh, min(c0 + 1, c1 - 1), N, e.tid);
    auto body = [&](const KV &b, int c) {
        __syncthreads();  // LDS free (previous chunk's readers are done)
        st.store_kv(e, b, c * C, N);
        __syncthreads();
        st.map(e, false, true, c * C, N);
        e.z_partials();
        e.state_update(acc);
        __syncthreads();
        if (e.tid < D) z += e.z_delta();
    };
    for (int c = c0; c < c1; c += 2) {
        body(b0, c);
        b0.template load<true>(Kh, Vh, min(c + 2, c1 - 1), N, e.tid);
        if (c + 1 < c1) body(b1, c + 1);
        b1.template load<true>(Kh, Vh, min(c + 3, c1 - 1), N, e.tid);
    }
}

// ---------------------------------------------------------------------------
// Phase B: outputs of chunks [c0, c1) starting from the state (S, z) of all
// earlier positions.  q0 already holds (or is loading) chunk c0's Q.
// kv_staged: chunk c0's phi(K), V are already in LDS.  advance_last: also
// advance the state over the last chunk (for the final state).  Loads run one
// chunk ahead.
// ---------------------------------------------------------------------------
template <typename T, int D, int M, int C, bool CAUSAL, bool PHI, typename OT, int DI = 0, typename TI = T>
__device__ __forceinline__ void phase_b(const Engine<T, D, M, C, PHI> &e, const TI *__restrict__ Qh,
                                        const TI *__restrict__ Kh, const TI *__restrict__ Vh,
                                        OT *__restrict__ Oh, int N, int c0, int c1, bool kv_staged,
                                        bool advance_last,
                                        typename ChunkStager<T, D, M, C, PHI, DI, TI>::QStage &q0,
                                        f32x4 (&S)[Cfg<T, D, M, C>::DT][Cfg<T, D, M, C>::MTW], float &z,
                                        bool poison, const ChunkStager<T, D, M, C, PHI, DI, TI> &st = {}) {
    // loads as in phase_a: one chunk ahead, unconditional (clamped)
    auto &q = q0;
    KVBuf<T, D, M, C, ChunkStager<T, D, M, C, PHI, DI, TI>::DQ, TI> b;
    if (CAUSAL && !kv_staged) b.template load<true>(Kh, Vh, c0, N, e.tid);
    for (int c = c0; c < c1; ++c) {
        const int row0 = c * C;
        const bool stage_kv = CAUSAL && !(kv_staged && c == c0);
        __syncthreads();  // LDS free
        st.store_q(e, q, row0, N);
        if (stage_kv) st.store_kv(e, b, row0, N);
        if (e.tid < D) e.set_z(z);
        __syncthreads();
        const int cn = min(c + 1, c1 - 1);
        q.template load<true>(Qh, cn * C, N, e.tid);
        if (CAUSAL) b.template load<true>(Kh, Vh, cn, N, e.tid);
        st.map(e, true, stage_kv, row0, N);
        if (CAUSAL) e.a_tiles();
        e.qz_rows();
        const bool adv = CAUSAL && (c + 1 < c1 || advance_last);
        if (adv) e.z_partials();
        __syncthreads();
        const float inv = e.template row_inv<CAUSAL>();
        f32x4 o[Cfg<T, D, M, C>::RT][Cfg<T, D, M, C>::MTW];
        Engine<T, D, M, C>::zero_out(o);
        if (CAUSAL) e.intra(o);
        e.readout(o, S, inv, Oh, row0, N, poison);
        if (adv) {
            e.state_update(S);
            if (e.tid < D) z += e.z_delta();
        }
    }
}

// ---------------------------------------------------------------------------
// Fused causal kernel: phase A, decoupled look-back over segments, phase B.
// With G == 1 there is no look-back and no workspace.
// ---------------------------------------------------------------------------
constexpr long kSpinLimit = 1L << 22;
// One-pass kernel: with at most this many segments per head no inclusive
// prefix is published; a look-back then sums every earlier aggregate (at most
// 15 slots, read from the device-wide cache), which costs less than the extra
// store and flag on every workgroup's path to its outputs.
constexpr int kOnePassInclusiveMinSegments = 16;

// Decoupled look-back of segment s > 0 of head bh (every thread of the
// workgroup calls it); the prefix of the earlier segments is added into pre /
// zpre.  Wavefront 0 polls the flags (one lane per segment, 64 at a time,
// relaxed loads) and the workgroup then sums the slots it names, in rounds:
//   in_order = false: one round, once it finds the nearest segment j* whose
//     inclusive prefix is published (segment 0's aggregate is its inclusive
//     prefix) with every aggregate between j* and s ready: incl(j*) +
//     agg(j*+1) + ... + agg(s-1);
//   in_order = true (no inclusive states are published): the aggregates of
//     segments 0 .. s-1 in segment order, each run of consecutive ready ones
//     as soon as its flags are seen, so the slots of segments that finished
//     early are read while later ones still compute.
// Each round passes (first segment + 1, count | inclusive bit) through two LDS
// words; rounds alternate between sh_word[0..1] and [2..3] (wavefront 0 writes
// a pair again only after every wavefront has passed the barrier of the round
// in between).  One code path for both modes keeps one copy of the slot sums
// (and its registers) in the kernel.  Waits are bounded (kSpinLimit polls); on
// a timeout the error word of the workspace is set and false is returned.
template <typename T, int D, int M, int C, bool PHI>
__device__ __forceinline__ bool look_back(const Engine<T, D, M, C, PHI> &e, const FusedWs &ws, unsigned *sh_word, int bh,
                                          int s, int G_, unsigned ep,
                                          f32x4 (&pre)[Cfg<T, D, M, C>::DT][Cfg<T, D, M, C>::MTW], float &zpre,
                                          bool in_order) {
    using Gc = Cfg<T, D, M, C>;
    const size_t h0 = (size_t)bh * G_;
    const unsigned *fl = ws.flags + h0;
    int next = 0;  // in order: segments [0, next) summed
    for (int round = 0; next < s; ++round) {
        unsigned *word = sh_word + 2 * (round & 1);
        if (e.w == 0) {
            int from = -1, count = 0;
            bool incl_first = false;
            int base = s - 1;  // inclusive mode: the newest segment of the polled window
            long spins = 0;
            // header word 4, when the host has set it, caps the polls (tests of the give-up path)
            const unsigned cap = __hip_atomic_load(&ws.hdr[kWsPollCapWord], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const long limit = cap != 0u ? (long)cap : kSpinLimit;
            while (true) {
                const int j = in_order ? next + e.lane : base - e.lane;
                const bool valid = in_order ? j < s : j >= 0;
                unsigned f = 0u;
                if (valid) f = __hip_atomic_load(fl + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const bool ok = valid && (f & ~3u) == ep && (f & 3u) != 0u;
                const unsigned long long okm = __ballot(ok);
                if (in_order) {
                    if (okm & 1ull) {  // lanes 0 .. count-1 ready
                        from = next;
                        count = okm == ~0ull ? 64 : __builtin_ctzll(~okm);
                        break;
                    }
                } else {
                    const bool inc = ok && ((f & 3u) == 2u || j == 0);
                    const unsigned long long incm = __ballot(inc);
                    if (incm != 0ull) {
                        const int first = __builtin_ctzll(incm);
                        const unsigned long long need = first == 63 ? ~0ull : ((1ull << (first + 1)) - 1ull);
                        if ((okm & need) == need) {
                            from = base - first;
                            count = s - from;
                            incl_first = from != 0;
                            break;
                        }
                    } else if (okm == ~0ull) {
                        base -= 64;  // 64 aggregates ready, none inclusive: look further back
                        continue;
                    }
                }
                if (++spins > limit) {
                    if (e.lane == 0)
                        __hip_atomic_store(&ws.hdr[kWsErrorWord], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    from = -1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (e.lane == 0) {
                word[0] = (unsigned)(from + 1);
                word[1] = (unsigned)count | (incl_first ? 0x80000000u : 0u);
            }
        }
        __syncthreads();
        const int from = (int)word[0] - 1;
        if (from < 0) return false;
        const int count = (int)(word[1] & 0x7fffffffu);
        const bool incl_first = (word[1] >> 31) != 0u;
        e.state_add_slots(pre, zpre, (incl_first ? ws.incl : ws.agg) + (h0 + from) * Gc::EP, ws.agg + h0 * Gc::EP,
                          from + 1, from + count);
        next = from + count;
    }
    return true;
}

// Publish the inclusive prefix pre + acc of segment `my` (NaN after a failed look-back).
template <typename T, int D, int M, int C, bool PHI>
__device__ __forceinline__ void publish_inclusive(const Engine<T, D, M, C, PHI> &e, const FusedWs &ws, size_t my,
                                                  unsigned ep,
                                                  const f32x4 (&pre)[Cfg<T, D, M, C>::DT][Cfg<T, D, M, C>::MTW],
                                                  float zpre,
                                                  const f32x4 (&acc)[Cfg<T, D, M, C>::DT][Cfg<T, D, M, C>::MTW],
                                                  float zacc, bool failed) {
    using Gc = Cfg<T, D, M, C>;
    f32x4 inc[Gc::DT][Gc::MTW];
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int dt = 0; dt < Gc::DT; ++dt)
#pragma unroll
        for (int i = 0; i < Gc::MTW; ++i) {
            inc[dt][i] = pre[dt][i] + acc[dt][i];
            if (failed) inc[dt][i] = f32x4{nan, nan, nan, nan};
        }
    e.slot_store(inc, failed ? nan : zpre + zacc, ws.incl + my * Gc::EP);
    e.publish_flag(&ws.flags[my], ep | 2u);
}

// Called by the last segment of every head once its look-back is done.  Every
// segment of that head has then read the epoch: the look-back saw a flag tagged
// with it from each earlier segment, directly or through an inclusive state
// (published only after that segment's own look-back saw the flags before it).
// So when the last of the n_heads heads has counted, no workgroup of
// the call will read the epoch again: that one resets the counter and advances
// the epoch (every flag of the call becomes stale).  One atomic per head instead
// of one per workgroup.
__device__ __forceinline__ void finish_call(const FusedWs &ws, unsigned epoch, unsigned n_heads) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned done = atomicAdd(&ws.hdr[1], 1u);
        if (done == n_heads - 1u) {
            __hip_atomic_store(&ws.hdr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ws.hdr[2], epoch + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// DI > 0: raw rows DI wide (type TI) mapped to random features while staged,
// as in the one-pass kernel.
template <typename T, int D, int M, int C, bool PHI = true, typename OT = float, int DI = 0, typename TI = T>
__global__ __launch_bounds__((Cfg<T, D, M, C>::THREADS), (Cfg<T, D, M, C>::MIN_WG)) void fused_causal_kernel(
    const TI *__restrict__ Q, const TI *__restrict__ K, const TI *__restrict__ V, OT *__restrict__ out, void *ws_raw,
    int BH, int N, int G_, int CPS, float *__restrict__ S_out, float *__restrict__ z_out, const float *S_in,
    const float *z_in, const float *__restrict__ W, int fkind, int fnorm) {
    using Gc = Cfg<T, D, M, C>;
    using En = Engine<T, D, M, C, PHI>;
    using St = ChunkStager<T, D, M, C, PHI, DI, TI>;
    constexpr int DQ = St::DQ;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Gc::bytes];
    __shared__ __attribute__((aligned(16))) float sfeat[St::FEAT ? St::FL::nRaw + St::FL::nW : 4];
    __shared__ unsigned sh_word[4];
    En e(smem);
    const int tid = e.tid;
    St st;
    st.init(sfeat, W, fkind, fnorm, tid);

    // Work item: block b -> segment b / BH of head b % BH.  Workgroups are
    // dispatched in block order, so a workgroup only ever waits on segments of
    // smaller block index, which are resident or finished; the waits are also
    // bounded (kSpinLimit) and a timeout poisons the outputs instead of hanging.
    const int bh = (int)(blockIdx.x % (unsigned)BH);
    const int s = (int)(blockIdx.x / (unsigned)BH);
    unsigned epoch = 0;
    FusedWs ws(ws_raw, BH, G_ > 1 ? G_ : 1, Gc::E);
    if (G_ > 1) {
        if (tid == 0) sh_word[1] = __hip_atomic_load(&ws.hdr[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        epoch = sh_word[1];
    }
    const unsigned ep = (epoch & 0x3fffffffu) << 2;

    const int n_chunks = (N + C - 1) / C;
    const int c0 = s * CPS, c1 = min(c0 + CPS, n_chunks);
    const TI *Qh = Q + (size_t)bh * N * DQ;
    const TI *Kh = K + (size_t)bh * N * DQ;
    const TI *Vh = V + (size_t)bh * N * M;
    OT *Oh = out + (size_t)bh * N * M;

    e.clear_a();

    f32x4 acc[Gc::DT][Gc::MTW];
    En::zero_state(acc);
    float zacc = 0.0f;
    const bool last = s == G_ - 1;
    const bool want_final = S_out != nullptr;
    const bool run_a = G_ > 1 && (!last || want_final);
    if (run_a) phase_a(e, Kh, Vh, N, c0, c1, acc, zacc, st);
    const size_t my = (size_t)bh * G_ + s;
    // Prefix of the segment: the carried initial state (segment 0, when given),
    // later the look-back's sum of the earlier segments.
    f32x4 pre[Gc::DT][Gc::MTW];
    En::zero_state(pre);
    float zpre = 0.0f;
    const bool init = S_in != nullptr && s == 0;
    if (init) e.state_add(pre, zpre, S_in + (size_t)bh * D * M, z_in + (size_t)bh * D);
    // publish the segment aggregate (segment 0: with the initial state, so that
    // it stays the inclusive prefix) before any other load is in flight (the
    // publication waits for every outstanding memory operation of the wave)
    if (G_ > 1 && !last) {
        if (init) {
            f32x4 a0[Gc::DT][Gc::MTW];
#pragma unroll
            for (int dt = 0; dt < Gc::DT; ++dt)
#pragma unroll
                for (int i = 0; i < Gc::MTW; ++i) a0[dt][i] = acc[dt][i] + pre[dt][i];
            e.slot_store(a0, zacc + zpre, ws.agg + my * Gc::EP);
        } else {
            e.slot_store(acc, zacc, ws.agg + my * Gc::EP);
        }
        e.publish_flag(&ws.flags[my], ep | 1u);
    }

    typename St::QStage stQ;
    stQ.template load<true>(Qh, c0 * C, N, tid);

    // A one-chunk segment still holds its phi(K), V in LDS: form A and the
    // intra-chunk term now, while earlier segments may still be publishing.
    f32x4 o[Gc::RT][Gc::MTW];
    En::zero_out(o);
    const bool single = run_a && (c1 - c0 == 1);
    if (single) {
        st.store_q(e, stQ, c0 * C, N);
        __syncthreads();
        st.map(e, true, false, c0 * C, N);
        e.a_tiles();
        __syncthreads();
        e.intra(o);
    }

    bool failed = false;
    if (G_ > 1 && s > 0) {
        failed = !look_back(e, ws, sh_word, bh, s, G_, ep, pre, zpre, false);
        if (!last) publish_inclusive(e, ws, (size_t)bh * G_ + s, ep, pre, zpre, acc, zacc, failed);
    }
    if (G_ > 1 && last && want_final) {
        f32x4 fin[Gc::DT][Gc::MTW];
#pragma unroll
        for (int dt = 0; dt < Gc::DT; ++dt)
#pragma unroll
            for (int i = 0; i < Gc::MTW; ++i) {
                fin[dt][i] = pre[dt][i] + acc[dt][i];
                if (failed) fin[dt][i] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
            }
        e.state_store(fin, failed ? __builtin_nanf("") : zpre + zacc, S_out + (size_t)bh * D * M,
                      z_out + (size_t)bh * D);
    }

    if (single) {
        // the rest of the one-chunk segment: normaliser and the inter-chunk term
        if (tid < D) e.set_z(zpre);
        __syncthreads();
        e.qz_rows();
        __syncthreads();
        const float inv = e.template row_inv<true>();
        e.readout(o, pre, inv, Oh, c0 * C, N, failed);
    } else {
        phase_b<T, D, M, C, true, PHI, OT, DI, TI>(e, Qh, Kh, Vh, Oh, N, c0, c1, false, G_ == 1 && want_final, stQ,
                                                   pre, zpre, failed, st);
        if (G_ == 1 && want_final) e.state_store(pre, zpre, S_out + (size_t)bh * D * M, z_out + (size_t)bh * D);
    }

    if (G_ > 1 && last) finish_call(ws, epoch, (unsigned)BH);
}

// ---------------------------------------------------------------------------
// One-pass causal kernel, for segments of at most kOnePassChunks chunks.
// The workgroup reads its segment once.  Per chunk it forms A, the intra-chunk
// term and phi(Q_c) times the state summed so far inside the segment, keeps
// the unnormalised rows in registers (and phi(Q_c) and the partial
// denominators in LDS), and advances the segment-local state.  It then
// publishes the local state (the segment aggregate), looks back for the
// prefix (S_p, z_p) of the earlier segments and finishes every row:
//   out = (o + phi(q) S_p) / (den + phi(q) . z_p).
// Same workspace, flags and epoch protocol as the fused kernel.
// ---------------------------------------------------------------------------
constexpr int kOnePassChunks = 4;

// LDS: phi(Q) of the whole segment [ROWS][LQ] at the start, its last chunk
// doubling as the engine's phi(Q) tile (the engine's layout starts at
// `shift`), then the partial denominators and phi(q).z_prefix of every row.
// ---------------------------------------------------------------------------
// Random features fused into the staging of Q and K (page "Stable, Fast and
// Accurate: Kernelized Attention with Relative Positional Encoding", Proposed
// method and Main findings: PRF and TRF feature maps, feature dimension F).  The
// raw q and k rows of a chunk (DI wide, fp32) are staged in LDS; the projections
// x W^T run on MFMA with W staged in LDS once per workgroup (rows past the number
// of projections zero); then kind 1 (PRF): exp(w . x - |x|^2 / 2) / sqrt(F),
// kind 2 (TRF, P = F / 2 projections): exp(|x|^2 / 2) / sqrt(P) times sin (column
// p) and cos (column P + p); norm: rows scaled to unit length first.  Rows at or
// beyond N get zero features (they must add nothing to the sums).
template <typename T, int D, int M, int C>
struct OnePassLds {
    using Gc = Cfg<T, D, M, C>;
    static constexpr int ROWS = kOnePassChunks * C;
    static constexpr size_t shift = (size_t)(kOnePassChunks - 1) * C * Gc::LQ * sizeof(T);
    static_assert(shift % 16 == 0, "phi(Q) rows keep 16-byte alignment");
    static constexpr size_t oDen = ((shift + Gc::bytes + 15) / 16) * 16;
    static constexpr size_t oQz = oDen + ROWS * sizeof(float);
    static constexpr size_t bytes = oQz + ROWS * sizeof(float);
    // every workgroup the planner places on one CU must fit
    static constexpr bool fits = (bytes + 64) * Gc::MIN_WG <= kMaxLds;
};

// DI > 0: Q and K hold raw rows DI wide (element type TI: fp32 or bf16, V too)
// and the random-feature map (W, fkind, fnorm) is applied in fp32 while staging
// them (D is then the feature dimension F, the engine fp32).
template <typename T, int D, int M, int C, bool PHI = true, typename OT = float, int DI = 0, typename TI = T>
__global__ __launch_bounds__((Cfg<T, D, M, C>::THREADS), (Cfg<T, D, M, C>::MIN_WG)) void onepass_causal_kernel(
    const TI *__restrict__ Q, const TI *__restrict__ K, const TI *__restrict__ V, OT *__restrict__ out,
    void *ws_raw, int BH, int N, int G_, int CPS, float *__restrict__ S_out, float *__restrict__ z_out,
    const float *S_in, const float *z_in, const float *__restrict__ W, int fkind, int fnorm) {
    using Gc = Cfg<T, D, M, C>;
    using L1 = OnePassLds<T, D, M, C>;
    using En = Engine<T, D, M, C, PHI>;
    constexpr int NC = kOnePassChunks;
    constexpr bool FEAT = DI > 0;
    constexpr int DQ = FEAT ? DI : D;  // width of the Q, K rows in memory
    using FL = FeatLds<FEAT ? DI : 16, D, C>;
    static_assert(!FEAT || (std::is_same<T, float>::value && !PHI), "fused features: fp32 engine, no elu map");
    static_assert(FEAT || std::is_same<TI, T>::value, "raw rows of another type only with fused features");
    __shared__ __attribute__((aligned(16))) unsigned char smem[L1::bytes];
    __shared__ __attribute__((aligned(16))) float sfeat[FEAT ? FL::nRaw + FL::nW : 4];
    __shared__ unsigned sh_word[4];
    En e(smem + L1::shift);
    T *const sQs = reinterpret_cast<T *>(smem);
    float *const sden = reinterpret_cast<float *>(smem + L1::oDen);
    float *const sqzs = reinterpret_cast<float *>(smem + L1::oQz);
    const int tid = e.tid;

    // block b -> segment b / BH of head b % BH (dispatch order, as in the fused kernel)
    const int bh = (int)(blockIdx.x % (unsigned)BH);
    const int s = (int)(blockIdx.x / (unsigned)BH);
    unsigned epoch = 0;
    FusedWs ws(ws_raw, BH, G_ > 1 ? G_ : 1, Gc::E);
    if (G_ > 1) {
        if (tid == 0) sh_word[1] = __hip_atomic_load(&ws.hdr[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        epoch = sh_word[1];
    }
    const unsigned ep = (epoch & 0x3fffffffu) << 2;

    const int n_chunks = (N + C - 1) / C;
    const int c0 = s * CPS;
    const int nc = min(CPS, n_chunks - c0);  // 1 .. NC (the planner guarantees it)
    const TI *Qh = Q + (size_t)bh * N * DQ;
    const TI *Kh = K + (size_t)bh * N * DQ;
    const TI *Vh = V + (size_t)bh * N * M;
    OT *Oh = out + (size_t)bh * N * M;
    const bool last = s == G_ - 1;
    const bool want_final = S_out != nullptr;
    float *const sRawQ = sfeat, *const sRawK = sfeat + C * FL::LX, *const sW = sfeat + FL::nRaw;
    const int P = fkind == 2 ? D / 2 : D;  // projections (fused features)
    if constexpr (FEAT) {
        // W once per workgroup, rows past P zero
        for (int x = tid; x < FL::WROWS * (DI / 4); x += Gc::THREADS) {
            const int f = x / (DI / 4), c4 = (x % (DI / 4)) * 4;
            f32x4 v = zero4();
            if (f < P) v = *reinterpret_cast<const f32x4 *>(W + (size_t)f * DI + c4);
            *reinterpret_cast<f32x4 *>(sW + f * FL::LX + c4) = v;
        }
    }

    e.clear_a();
    f32x4 S[Gc::DT][Gc::MTW];
    En::zero_state(S);
    float z = 0.0f;
    f32x4 o[NC][Gc::RT][Gc::MTW];
#pragma unroll
    for (int j = 0; j < NC; ++j) En::zero_out(o[j]);
    // SNAP: the local state after each chunk is kept in registers and every
    // chunk's read-out phi(Q_c) (prefix + local state) runs once, after the
    // look-back, instead of a local read-out in the chunk loop plus a prefix
    // correction afterwards (one state product per chunk fewer, off the chunk
    // loop).  Used where the copies fit the register budget.
    constexpr bool SNAP = C >= 32 && Gc::DT * Gc::MTW * (NC - 1) <= 12;
    f32x4 snap[SNAP ? NC - 1 : 1][Gc::DT][Gc::MTW];

    // loads one chunk ahead, unconditional (clamped to the segment's last chunk)
    // so the compiler's wait counts stay exact (see phase_a)
    const int clast = c0 + nc - 1;
    Stage<TI, C, DQ, Gc::THREADS> q;
    KVBuf<T, D, M, C, DQ, TI> b;
    q.load(Qh, c0 * C, N, tid);
    b.load(Kh, Vh, c0, N, tid);
    auto step = [&](int j, f32x4 (&oj)[Gc::RT][Gc::MTW]) {
        const int c = c0 + j, row0 = c * C;
        __syncthreads();  // sK, sV, sA, side arrays free
        e.sQ = sQs + j * C * Gc::LQ;
        if constexpr (FEAT) {
            // raw rows to LDS, then the features of q and k into the engine's tiles
            q.store_natural_f32(sRawQ, FL::LX, row0, N, tid);
            b.k.store_natural_f32(sRawK, FL::LX, row0, N, tid);
            b.v.store_natural_f32(e.sV, Gc::LV, row0, N, tid);
            if (tid < D) e.set_z(z);
            __syncthreads();
            const int PT = (P + 15) / 16, jobs = 2 * Gc::RT * PT;
            for (int jb = e.w; jb < jobs; jb += Gc::NW) {
                const int t = jb / (Gc::RT * PT), rt = (jb % (Gc::RT * PT)) / PT, pt = jb % PT;
                feature_job<DI, D, C>(t == 0 ? sRawQ : sRawK, sW, t == 0 ? e.sQ : e.sK, Gc::LQ, rt, pt, P, fkind,
                                      fnorm != 0, row0, N, e.lane);
            }
        } else {
            e.store_q(q, row0, N);
            e.store_kv(b.k, b.v, row0, N);
            if (tid < D) e.set_z(z);
        }
        __syncthreads();
        if (j + 1 < NC) {  // compile-time: no load past the last possible step
            q.load(Qh, min(c + 1, clast) * C, N, tid);
            b.load(Kh, Vh, min(c + 1, clast), N, tid);
        }
        e.a_tiles();
        e.qz_rows();
        // the last segment needs its local state only for the final state
        const bool adv = j + 1 < nc || !last || want_final;
        if (adv) e.z_partials();
        __syncthreads();
        if (e.w == 0 && e.lane < C) sden[j * C + e.lane] = e.template row_den<true>();
        e.intra(oj);
        if (!SNAP && j > 0) e.readout_mma(oj, S);
        if (adv) {
            e.state_update(S);
            if (tid < D) z += e.z_delta();
        }
        if constexpr (SNAP) {
            if (j + 1 < NC) {
#pragma unroll
                for (int dt = 0; dt < Gc::DT; ++dt)
#pragma unroll
                    for (int i = 0; i < Gc::MTW; ++i) snap[j][dt][i] = S[dt][i];
            }
        }
    };
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        if (j < nc) step(j, o[j]);
    }

    const size_t my = (size_t)bh * G_ + s;
    // prefix: the carried initial state for segment 0 (when given), else the look-back's
    f32x4 pre[Gc::DT][Gc::MTW];
    En::zero_state(pre);
    float zpre = 0.0f;
    const bool init = S_in != nullptr && s == 0;
    if (init) e.state_add(pre, zpre, S_in + (size_t)bh * D * M, z_in + (size_t)bh * D);
    if (G_ > 1 && !last) {
        if (init) {
            f32x4 a0[Gc::DT][Gc::MTW];
#pragma unroll
            for (int dt = 0; dt < Gc::DT; ++dt)
#pragma unroll
                for (int i = 0; i < Gc::MTW; ++i) a0[dt][i] = S[dt][i] + pre[dt][i];
            e.slot_store(a0, z + zpre, ws.agg + my * Gc::EP);
        } else {
            e.slot_store(S, z, ws.agg + my * Gc::EP);
        }
        e.publish_flag(&ws.flags[my], ep | 1u);
    }
    bool failed = false;
    const bool has_prefix = (G_ > 1 && s > 0) || init;
    if (G_ > 1 && s > 0) {
        const bool in_order = G_ <= kOnePassInclusiveMinSegments;
        failed = !look_back(e, ws, sh_word, bh, s, G_, ep, pre, zpre, in_order);
        if (!in_order && !last) publish_inclusive(e, ws, my, ep, pre, zpre, S, z, failed);
    }
    if (last && want_final) {
        f32x4 fin[Gc::DT][Gc::MTW];
#pragma unroll
        for (int dt = 0; dt < Gc::DT; ++dt)
#pragma unroll
            for (int i = 0; i < Gc::MTW; ++i) {
                fin[dt][i] = pre[dt][i] + S[dt][i];
                if (failed) fin[dt][i] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
            }
        e.state_store(fin, failed ? __builtin_nanf("") : zpre + z, S_out + (size_t)bh * D * M,
                      z_out + (size_t)bh * D);
    }

    // finish the rows with the prefix
    if (has_prefix) {
        if (tid < D) e.set_z(zpre);
        __syncthreads();
        for (int j = 0; j < nc; ++j) {
            e.sQ = sQs + j * C * Gc::LQ;
            e.qz_rows_to(sqzs + j * C);
        }
    }
    __syncthreads();  // sden, sqzs visible to every wavefront
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        if (j < nc) {
            float inv = 0.0f;
            if (e.lane < C) inv = 1.0f / (sden[j * C + e.lane] + (has_prefix ? sqzs[j * C + e.lane] : 0.0f));
            if constexpr (SNAP) {
                if (has_prefix || j > 0) {
                    f32x4 Sj[Gc::DT][Gc::MTW];
#pragma unroll
                    for (int dt = 0; dt < Gc::DT; ++dt)
#pragma unroll
                        for (int i = 0; i < Gc::MTW; ++i) Sj[dt][i] = j > 0 ? pre[dt][i] + snap[j - 1][dt][i] : pre[dt][i];
                    e.sQ = sQs + j * C * Gc::LQ;
                    e.readout_mma(o[j], Sj);
                }
            } else if (has_prefix) {
                e.sQ = sQs + j * C * Gc::LQ;
                e.readout_mma(o[j], pre);
            }
            e.store_rows(o[j], inv, Oh, (c0 + j) * C, N, failed);
        }
    }
    if (G_ > 1 && last) finish_call(ws, epoch, (unsigned)BH);
}

// ---------------------------------------------------------------------------
// Stage kernels (explicit three-step form; also the non-causal path).
// Stage workspace: [BH][G + 1][E]; slot s = state of segment s, later its
// exclusive prefix; slot G = total.
// ---------------------------------------------------------------------------
// DI > 0 (both stage kernels): raw rows DI wide (type TI) mapped to random
// features while staged, as in the causal kernels.
template <typename T, int D, int M, int C, bool PHI = true, int DI = 0, typename TI = T>
__global__ __launch_bounds__((Cfg<T, D, M, C>::THREADS), (Cfg<T, D, M, C>::MIN_WG)) void seg_state_kernel(
    const TI *__restrict__ K, const TI *__restrict__ V, float *__restrict__ ws, int N, int G_, int CPS, int nstates,
    const float *__restrict__ W = nullptr, int fkind = 0, int fnorm = 0) {
    using Gc = Cfg<T, D, M, C>;
    using St = ChunkStager<T, D, M, C, PHI, DI, TI>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Gc::bytes];
    __shared__ __attribute__((aligned(16))) float sfeat[St::FEAT ? St::FL::nRaw + St::FL::nW : 4];
    Engine<T, D, M, C, PHI> e(smem);
    St st;
    st.init(sfeat, W, fkind, fnorm, e.tid);
    const int bh = blockIdx.x / nstates, s = blockIdx.x % nstates;
    const int n_chunks = (N + C - 1) / C;
    const int c0 = s * CPS, c1 = min(c0 + CPS, n_chunks);
    f32x4 acc[Gc::DT][Gc::MTW];
    Engine<T, D, M, C>::zero_state(acc);
    float z = 0.0f;
    phase_a(e, K + (size_t)bh * N * St::DQ, V + (size_t)bh * N * M, N, c0, c1, acc, z, st);
    e.state_store(acc, z, ws + ((size_t)bh * (G_ + 1) + s) * Gc::E);
}

template <typename T, int D, int M, int C, bool CAUSAL, bool PHI = true, typename OT = float, int DI = 0,
          typename TI = T>
__global__ __launch_bounds__((Cfg<T, D, M, C>::THREADS), (Cfg<T, D, M, C>::MIN_WG)) void seg_output_kernel(
    const TI *__restrict__ Q, const TI *__restrict__ K, const TI *__restrict__ V, OT *__restrict__ out,
    const float *__restrict__ ws, int N, int G_, int CPS, float *__restrict__ S_out, float *__restrict__ z_out,
    const float *__restrict__ W = nullptr, int fkind = 0, int fnorm = 0) {
    using Gc = Cfg<T, D, M, C>;
    using St = ChunkStager<T, D, M, C, PHI, DI, TI>;
    constexpr int DQ = St::DQ;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Gc::bytes];
    __shared__ __attribute__((aligned(16))) float sfeat[St::FEAT ? St::FL::nRaw + St::FL::nW : 4];
    Engine<T, D, M, C, PHI> e(smem);
    St st;
    st.init(sfeat, W, fkind, fnorm, e.tid);
    const int bh = blockIdx.x / G_, s = blockIdx.x % G_;
    const int n_chunks = (N + C - 1) / C;
    const int c0 = s * CPS, c1 = min(c0 + CPS, n_chunks);
    const TI *Qh = Q + (size_t)bh * N * DQ;
    f32x4 S[Gc::DT][Gc::MTW];
    Engine<T, D, M, C>::zero_state(S);
    float z = 0.0f;
    if (CAUSAL) {
        if (s > 0) e.state_add(S, z, ws + ((size_t)bh * (G_ + 1) + s) * Gc::E);
    } else {
        e.state_add(S, z, ws + ((size_t)bh * (G_ + 1) + G_) * Gc::E);
    }
    if (CAUSAL) e.clear_a();
    typename St::QStage stQ;
    stQ.load(Qh, c0 * C, N, e.tid);
    const bool fin = CAUSAL && S_out != nullptr && s == G_ - 1;
    phase_b<T, D, M, C, CAUSAL, PHI, OT, DI, TI>(e, Qh, K + (size_t)bh * N * DQ, V + (size_t)bh * N * M,
                                                 out + (size_t)bh * N * M, N, c0, c1, false, fin, stQ, S, z, false, st);
    if (fin) e.state_store(S, z, S_out + (size_t)bh * D * M, z_out + (size_t)bh * D);
}

}  // namespace la

#include "la_engine32.hpp"

namespace la {

// ---------------------------------------------------------------------------
// Host-side launchers (instantiated per element type in la_prefill_*.hip).
// ---------------------------------------------------------------------------
template <typename T, int D, int M, int C, bool PHI = true, typename OT = float>
hipError_t run_fused(const void *Q, const void *K, const void *V, void *out, void *ws, int BH, int N, int G_,
                     int CPS, float *S_out, float *z_out, const float *S_in, const float *z_in, hipStream_t stream) {
    using Gc = Cfg<T, D, M, C>;
    if constexpr (!Gc::fits) {
        return hipErrorInvalidValue;
    } else {
        if (BH <= 0 || G_ <= 0) return hipSuccess;
        const unsigned grid = (unsigned)(G_ > 1 ? BH * G_ : BH);
        if constexpr (std::is_same<T, bf16>::value && D == 128 && M == 128 && C == 64 && PHI) {
            // bf16, D = M = 128, chunk 64: the engine on 32x32x16 tiles
            hipLaunchKernelGGL((fused_causal32_kernel<OT>), dim3(grid), dim3(Gc::THREADS), 0, stream, (const bf16 *)Q,
                               (const bf16 *)K, (const bf16 *)V, (OT *)out, ws, BH, N, G_, CPS, S_out, z_out, S_in,
                               z_in);
            return hipGetLastError();
        }
        hipLaunchKernelGGL((fused_causal_kernel<T, D, M, C, PHI, OT>), dim3(grid), dim3(Gc::THREADS), 0, stream, (const T *)Q,
                           (const T *)K, (const T *)V, (OT *)out, ws, BH, N, G_, CPS, S_out, z_out, S_in, z_in, nullptr,
                           0, 0);
        return hipGetLastError();
    }
}

template <typename T, int D, int M, int C, bool PHI = true, typename OT = float>
hipError_t run_onepass(const void *Q, const void *K, const void *V, void *out, void *ws, int BH, int N, int G_,
                       int CPS, float *S_out, float *z_out, const float *S_in, const float *z_in,
                       hipStream_t stream) {
    using Gc = Cfg<T, D, M, C>;
    if constexpr (!(Gc::fits && OnePassLds<T, D, M, C>::fits)) {
        return hipErrorInvalidValue;
    } else {
        if (BH <= 0 || G_ <= 0) return hipSuccess;
        if (CPS < 1 || CPS > kOnePassChunks) return hipErrorInvalidValue;
        hipLaunchKernelGGL((onepass_causal_kernel<T, D, M, C, PHI, OT>), dim3((unsigned)(BH * G_)), dim3(Gc::THREADS), 0,
                           stream, (const T *)Q, (const T *)K, (const T *)V, (OT *)out, ws, BH, N, G_, CPS, S_out, z_out,
                           S_in, z_in, nullptr, 0, 0);
        return hipGetLastError();
    }
}

// The one-pass kernel with the random-feature map fused (fp32 q, k rows DI wide,
// F features, W [P][DI]); see onepass_causal_kernel.
template <int DI, int F, int M, int C>
constexpr bool onepass_features_fit() {
    using Gc = Cfg<float, F, M, C>;
    return Gc::fits && OnePassLds<float, F, M, C>::fits &&
           (OnePassLds<float, F, M, C>::bytes + FeatLds<DI, F, C>::bytes + 64) * Gc::MIN_WG <= kMaxLds;
}

template <int DI, int F, int M, int C, typename TI = float>
hipError_t run_onepass_features(const void *Q, const void *K, const void *V, const float *W, int fkind, int fnorm,
                                float *out, void *ws, int BH, int N, int G_, int CPS, float *S_out, float *z_out,
                                const float *S_in, const float *z_in, hipStream_t stream) {
    using Gc = Cfg<float, F, M, C>;
    if constexpr (!onepass_features_fit<DI, F, M, C>()) {
        return hipErrorInvalidValue;
    } else {
        if (BH <= 0 || G_ <= 0) return hipSuccess;
        if (CPS < 1 || CPS > kOnePassChunks) return hipErrorInvalidValue;
        hipLaunchKernelGGL((onepass_causal_kernel<float, F, M, C, false, float, DI, TI>), dim3((unsigned)(BH * G_)),
                           dim3(Gc::THREADS), 0, stream, (const TI *)Q, (const TI *)K, (const TI *)V, out, ws,
                           BH, N, G_, CPS, S_out, z_out, S_in, z_in, W, fkind, fnorm);
        return hipGetLastError();
    }
}

// Non-causal attention over random features (the stage path: segment states,
// their scan, outputs), raw rows of type TI mapped in both stage kernels.
template <int DI, int F, int M, int C>
constexpr bool stage_features_fit() {
    using Gc = Cfg<float, F, M, C>;
    return Gc::fits && Gc::bytes + FeatLds<DI, F, C>::bytes + 64 <= kMaxLds;
}

template <int DI, int F, int M, int C, typename TI = float>
hipError_t run_noncausal_features(const void *Q, const void *K, const void *V, const float *W, int fkind, int fnorm,
                                  float *out, float *ws, int BH, int N, int G_, int CPS, hipStream_t stream) {
    using Gc = Cfg<float, F, M, C>;
    if constexpr (!stage_features_fit<DI, F, M, C>()) {
        return hipErrorInvalidValue;
    } else {
        if (BH <= 0 || G_ <= 0) return hipSuccess;
        hipLaunchKernelGGL((seg_state_kernel<float, F, M, C, false, DI, TI>), dim3((unsigned)(BH * G_)),
                           dim3(Gc::THREADS), 0, stream, (const TI *)K, (const TI *)V, ws, N, G_, CPS, G_, W, fkind,
                           fnorm);
        hipError_t e = hipGetLastError();
        if (e == hipSuccess) e = prefill_scan(ws, BH, F, M, G_, G_, nullptr, nullptr, stream);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((seg_output_kernel<float, F, M, C, false, false, float, DI, TI>), dim3((unsigned)(BH * G_)),
                           dim3(Gc::THREADS), 0, stream, (const TI *)Q, (const TI *)K, (const TI *)V, out, ws, N, G_,
                           CPS, nullptr, nullptr, W, fkind, fnorm);
        return hipGetLastError();
    }
}

template <typename T, int D, int M, int C, bool PHI = true>
hipError_t run_states(const void *K, const void *V, float *ws, int BH, int N, int G_, int CPS, int nstates,
                      hipStream_t stream) {
    using Gc = Cfg<T, D, M, C>;
    if constexpr (!Gc::fits) {
        return hipErrorInvalidValue;
    } else {
        if (nstates <= 0 || BH <= 0) return hipSuccess;
        hipLaunchKernelGGL((seg_state_kernel<T, D, M, C, PHI>), dim3((unsigned)(BH * nstates)), dim3(Gc::THREADS), 0, stream,
                           (const T *)K, (const T *)V, ws, N, G_, CPS, nstates);
        return hipGetLastError();
    }
}

template <typename T, int D, int M, int C, bool PHI = true, typename OT = float>
hipError_t run_outputs(const void *Q, const void *K, const void *V, void *out, const float *ws, int BH, int N,
                       int G_, int CPS, int causal, float *S_out, float *z_out, hipStream_t stream) {
    using Gc = Cfg<T, D, M, C>;
    if constexpr (!Gc::fits) {
        return hipErrorInvalidValue;
    } else {
        if (BH <= 0 || G_ <= 0) return hipSuccess;
        const dim3 grid((unsigned)(BH * G_)), block(Gc::THREADS);
        if (causal)
            hipLaunchKernelGGL((seg_output_kernel<T, D, M, C, true, PHI, OT>), grid, block, 0, stream, (const T *)Q,
                               (const T *)K, (const T *)V, (OT *)out, ws, N, G_, CPS, S_out, z_out);
        else
            hipLaunchKernelGGL((seg_output_kernel<T, D, M, C, false, PHI, OT>), grid, block, 0, stream, (const T *)Q,
                               (const T *)K, (const T *)V, (OT *)out, ws, N, G_, CPS, S_out, z_out);
        return hipGetLastError();
    }
}

// Every (D, M, C) the library instantiates: D, M in {16, 32, 64, 128}, C in {16, 32, 64}.
#define LA_FOR_C(D_, M_, X) X(D_, M_, 16) X(D_, M_, 32) X(D_, M_, 64)
#define LA_FOR_M(D_, X) LA_FOR_C(D_, 16, X) LA_FOR_C(D_, 32, X) LA_FOR_C(D_, 64, X) LA_FOR_C(D_, 128, X)
#define LA_FOR_ALL(X) LA_FOR_M(16, X) LA_FOR_M(32, X) LA_FOR_M(64, X) LA_FOR_M(128, X)

}  // namespace la
