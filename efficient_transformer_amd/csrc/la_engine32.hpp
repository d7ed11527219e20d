// The causal two-phase kernel for bf16 inputs with D = M = 128 and chunks of 64
// positions, on 32x32x16 MFMA tiles.
//
// Page "Transformers are RNNs" (Katharopoulos et al., 2020), Proposed method:
// the same chunked form of the causal sums as the generic engine
// (A = tril(phi(Q_c) phi(K_c)^T), num = A V_c + phi(Q_c) S, den = rowsum(A) +
// phi(Q_c) z, S += phi(K_c)^T V_c), with the state held in 32 x 32 blocks.  On
// gfx950 the bf16 32x32x16 MFMA does twice the work of a 16x16x32 one for about
// the same issue time, and each of its operands serves 32 rows or columns
// instead of 16, so the state update and the read-out need half the LDS operand
// bytes per product.
//
// Work split (eight wavefronts): wavefront w owns the state blocks of columns
// m in [32 mb, 32 mb + 32) (mb = w % 4) and rows d in the half dh = w / 4 of
// the 128 rows (two 32 x 32 blocks, t = 0, 1: rows 32 (2 dh + t) ..).  Its
// read-out of a chunk is therefore a partial sum over its 64 rows of d, for all
// 64 rows of the chunk; the two wavefronts of one column block add their
// partials through LDS: wavefront (mb, dh) finishes the chunk rows of half dh
// (adding its partner's partial and the intra-chunk term) and hands over the
// other half, read after the barrier that follows the products.  The phi(Q),
// phi(K), V tiles are double-buffered, so a chunk is staged beside the
// previous chunk's products: phase B takes two barriers per chunk, phase A
// one.
//
// Register layouts (lane l, h = l / 32, l32 = l % 32; value v of a 16-value
// accumulator): a 32 x 32 result holds row 8 (v / 4) + 4 h + v % 4 and column
// l32; an operand lane holds row (A) or column (B) l32 and the contraction slots
// 8 h .. 8 h + 7.  The read-out takes a state block's values 8 s .. 8 s + 7 as
// its A operand for contraction step s: they are the rows
// d = 32 db + 16 s + 4 h + {0..3} and + 8, so the phi(Q) operand reads the same
// two 4-element pieces of the query row.  The look-back and the published
// segment states reuse the generic engine's slot code: a slot holds the
// wavefront's values in its own lane order, which every workgroup of this kernel
// shares.
#pragma once

namespace la {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 r;
#pragma unroll
    for (int v = 0; v < 16; ++v) r[v] = 0.0f;
    return r;
}

struct Engine32 : Engine<bf16, 128, 128, 64, true> {
    using Base = Engine<bf16, 128, 128, 64, true>;
    using Gc = Cfg<bf16, 128, 128, 64>;
    static constexpr int D = 128, M = 128, C = 64;
    static_assert(Gc::NW == 8 && Gc::MTW == 1 && Gc::DT == 8, "eight wavefronts, one 16-column slice each");
    int mb, dh, h, l32;
    float *sx;  // hand-over tiles: [wavefront][4][64 lanes] f32x4

    __device__ __forceinline__ Engine32(unsigned char *smem, float *xchg) : Base(smem) {
        mb = w & 3;
        dh = w >> 2;
        h = lane >> 5;
        l32 = lane & 31;
        sx = xchg;
    }

    // 32x32x16 operand from a swizzled bf16 tile [keys][W]: lane l gets keys
    // kb + 8 h .. kb + 8 h + 7 of column col0 + l32 (two transposed reads, each
    // 16-lane group g covering columns col0 + 16 (g % 2) and keys + 8 (g / 2)).
    template <int W>
    __device__ __forceinline__ bf16x8 tr8x(const bf16 *tile, int kb, int col0) const {
        const int gg = lane >> 4;
        const int k0 = kb + 8 * (gg >> 1), c0 = col0 + 16 * (gg & 1);
        const bf16x4 lo = tr4<W>(tile, k0, c0, l16);
        const bf16x4 hi = tr4<W>(tile, k0 + 4, c0, l16);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }

    // S[own blocks] += phi(K_c)^T V_c
    __device__ __forceinline__ void state_update32(f32x16 (&S)[2]) const {
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
            const bf16x8 bv = tr8x<M>(sV, 16 * ks, 32 * mb);
#pragma unroll
            for (int t = 0; t < 2; ++t) S[t] = mma32_bf16(tr8x<D>(sK, 16 * ks, 32 * (2 * dh + t)), bv, S[t]);
        }
    }

    // the A operand of read-out step s of block t: the block's values 8 s .. 8 s + 7 in bf16
    static __device__ __forceinline__ bf16x8 state_operand(const f32x16 &S, int s) {
        return bf16x8{(bf16)S[8 * s + 0], (bf16)S[8 * s + 1], (bf16)S[8 * s + 2], (bf16)S[8 * s + 3],
                      (bf16)S[8 * s + 4], (bf16)S[8 * s + 5], (bf16)S[8 * s + 6], (bf16)S[8 * s + 7]};
    }
    // partial read-out over the own rows of d: P = (phi(Q)[rows 32 qb ..] S[own d, own m])^T
    __device__ __forceinline__ f32x16 readout_part(const bf16x8 (&sa)[2][2], int qb) const {
        f32x16 P = zero16();
        const int qrow = 32 * qb + l32;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int c = 32 * (2 * dh + t) + 16 * s + 4 * h;
                const bf16x4 q0 = rd4<D>(sQ, qrow, c);
                const bf16x4 q1 = rd4<D>(sQ, qrow, c + 8);
                P = mma32_bf16(sa[t][s], bf16x8{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]}, P);
            }
        return P;
    }

    // The chunk's work after its third barrier: the partial read-outs of both row
    // halves (the other half handed over through LDS), the intra-chunk term of the
    // own half, then the state update (adv) on the same V operands.  Returns the
    // own half's unnormalised rows.
    __device__ __forceinline__ f32x16 chunk_outputs(f32x16 (&S)[2], bool adv) const {
        bf16x8 sa[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s) sa[t][s] = state_operand(S[t], s);
        {
            const f32x16 Po = readout_part(sa, 1 - dh);
            f32x4 *dst = reinterpret_cast<f32x4 *>(sx) + (w * 4) * 64 + lane;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[j * 64] = f32x4{Po[4 * j], Po[4 * j + 1], Po[4 * j + 2], Po[4 * j + 3]};
        }
        f32x16 Pm = readout_part(sa, dh);
        const bf16 *arow = sA + (32 * dh + l32) * Gc::LA + 8 * h;
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
            const bf16x8 bv = tr8x<M>(sV, 16 * ks, 32 * mb);
            // keys of the own half's rows: 0 .. 32 dh + 31 (A is zero above the diagonal)
            if (ks <= 2 * dh + 1) Pm = mma32_bf16(bv, *reinterpret_cast<const bf16x8 *>(arow + 16 * ks), Pm);
            if (adv) {
#pragma unroll
                for (int t = 0; t < 2; ++t) S[t] = mma32_bf16(tr8x<D>(sK, 16 * ks, 32 * (2 * dh + t)), bv, S[t]);
            }
        }
        return Pm;
    }

    // Rows 32 dh .. 32 dh + 31 of the chunk at row0: own partial + the partner's
    // hand-over, times inv_q (the row's 1 / den), stored (after a barrier that
    // follows the partner's hand-over).  The finished 32 x 32 tile goes back into
    // the hand-over tile just read (only this wavefront uses it until the next
    // chunk's hand-over) as rows of 32 floats, 16-byte pieces XOR-swizzled by the
    // row, and is read back a row-piece per lane: every store instruction then
    // writes 8 rows of 128 contiguous bytes (nontemporal: written once, not
    // read).  LDS operations of one wavefront run in issue order; the fence keeps
    // the compiler from moving the reads first.
    template <typename OT>
    __device__ __forceinline__ void finish(const f32x16 &Pm, float inv_q, OT *__restrict__ Oh, int row0, int N,
                                           bool poison) const {
        f32x4 *tile = reinterpret_cast<f32x4 *>(sx) + ((w ^ 4) * 4) * 64;
        const float f = poison ? __builtin_nanf("") : inv_q;  // a poisoned call's rows are NaN
        f32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 x = tile[j * 64 + lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[j][r] = (Pm[4 * j + r] + x[r]) * f;
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // row q = l32 of the tile, columns 8 j + 4 h .. + 3: 16-byte piece 2 j + h
#pragma unroll
        for (int j = 0; j < 4; ++j) tile[l32 * 8 + ((2 * j + h) ^ (l32 & 7))] = v[j];
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const int p = lane & 7;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int q = 8 * k + (lane >> 3);
            const f32x4 y = tile[q * 8 + (p ^ (q & 7))];
            const int grow = row0 + 32 * dh + q;
            if (grow < N) {
                OT *dst = Oh + (size_t)grow * M + 32 * mb + 4 * p;
                if constexpr (std::is_same<OT, float>::value) {
                    __builtin_nontemporal_store(y, reinterpret_cast<f32x4 *>(dst));
                } else {
                    __builtin_nontemporal_store(bf16x4{(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]},
                                                reinterpret_cast<bf16x4 *>(dst));
                }
            }
        }
    }

    // state value v of block t <-> (d, m)
    __device__ __forceinline__ int srow(int t, int v) const {
        return 32 * (2 * dh + t) + 8 * (v >> 2) + 4 * h + (v & 3);
    }
    __device__ __forceinline__ int scol() const { return 32 * mb + l32; }
    __device__ __forceinline__ void state_store32(const f32x16 (&S)[2], float z, float *Sd, float *zd) const {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) Sd[srow(t, v) * M + scol()] = S[t][v];
        if (tid < D) zd[tid] = z;
    }
    __device__ __forceinline__ void state_add32(f32x16 (&S)[2], float &z, const float *Sd, const float *zd) const {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) S[t][v] += Sd[srow(t, v) * M + scol()];
        if (tid < D) z += zd[tid];
    }
    // the generic slot layout (f32x4 [DT][1]): entry 4 t + j holds values 4 j .. 4 j + 3 of block t
    static __device__ __forceinline__ void to4(const f32x16 (&S)[2], f32x4 (&X)[8][1]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                X[4 * t + j][0] = f32x4{S[t][4 * j], S[t][4 * j + 1], S[t][4 * j + 2], S[t][4 * j + 3]};
    }
    static __device__ __forceinline__ void from4(const f32x4 (&X)[8][1], f32x16 (&S)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[t][4 * j + r] = X[4 * t + j][0][r];
    }
};

// Phase A on the 32x32 engine: the segment's state over chunks [c0, c1).  Two
// register buffers (loads two chunks ahead, reloaded unconditionally with the
// chunk index clamped) and two LDS tile buffers with their own column-sum
// partials (e and e1, fixed per unrolled step): a step stages chunk c + 1 into
// the other buffer, then forms chunk c's column sums and state update; one
// barrier per chunk, after which chunk c's column sums are added.
__device__ __forceinline__ void phase_a32(const Engine32 &e, const Engine32 &e1, const bf16 *__restrict__ Kh,
                                          const bf16 *__restrict__ Vh, int N, int c0, int c1, f32x16 (&acc)[2],
                                          float &z) {
    using KV = KVBuf<bf16, 128, 128, 64>;
    constexpr int C = 64;
    KV b0, b1;
    b0.template load<true>(Kh, Vh, c0, N, e.tid);
    b1.template load<true>(Kh, Vh, min(c0 + 1, c1 - 1), N, e.tid);
    __syncthreads();
    e.store_kv(b0.k, b0.v, c0 * C, N);
    b0.template load<true>(Kh, Vh, min(c0 + 2, c1 - 1), N, e.tid);
    __syncthreads();
    // bn holds chunk c + 1 on entry and is reloaded with chunk c + 3
    auto step = [&](const Engine32 &cur, const Engine32 &nxt, KV &bn, int c, bool valid) {
        if (valid && c + 1 < c1) nxt.store_kv(bn.k, bn.v, (c + 1) * C, N);
        bn.template load<true>(Kh, Vh, min(c + 3, c1 - 1), N, e.tid);
        if (valid) {
            cur.z_partials();
            cur.state_update32(acc);
        }
        __syncthreads();
        if (valid && e.tid < 128) z += cur.z_delta();
    };
    for (int c = c0; c < c1; c += 2) {
        step(e, e1, b1, c, true);
        step(e1, e, b0, c + 1, c + 1 < c1);
    }
}

// Phase B on the 32x32 engine: outputs of chunks [c0, c1) from the state S of all
// earlier positions.  The phi(Q), phi(K), V tiles are double-buffered in LDS
// (e: buffer 0, e1: buffer 1, fixed per unrolled step so that every tile
// address stays a constant offset): a step stages chunk c + 1 into the other
// buffer and issues the loads of chunk c + 2, then forms chunk c's outputs and
// state update; after one barrier it stores chunk c's rows (the hand-over of
// the row halves is complete) and forms chunk c + 1's A tiles, phi(q) . z and
// column sums; a second barrier ends the step.  Two barriers per chunk, and
// the staging of one chunk sits beside the products of the previous one.
template <typename OT>
__device__ __forceinline__ void phase_b32(const Engine32 &e, const Engine32 &e1, const bf16 *__restrict__ Qh,
                                          const bf16 *__restrict__ Kh, const bf16 *__restrict__ Vh,
                                          OT *__restrict__ Oh, int N, int c0, int c1, bool advance_last,
                                          Stage<bf16, 64, 128, 512> &q, f32x16 (&S)[2], float &z, bool poison) {
    constexpr int C = 64;
    KVBuf<bf16, 128, 128, 64> b;
    b.template load<true>(Kh, Vh, c0, N, e.tid);
    // prologue: chunk c0 into buffer 0, its A tiles and sums
    __syncthreads();  // LDS free (phase A and the look-back are done with it)
    e.store_q(q, c0 * C, N);
    e.store_kv(b.k, b.v, c0 * C, N);
    if (e.tid < 128) e.set_z(z);
    {
        const int cn = min(c0 + 1, c1 - 1);
        q.template load<true>(Qh, cn * C, N, e.tid);
        b.template load<true>(Kh, Vh, cn, N, e.tid);
    }
    __syncthreads();
    e.a_tiles();
    e.qz_rows();
    if (c0 + 1 < c1 || advance_last) e.z_partials();
    __syncthreads();
    // step for chunk c (valid: c < c1; uniform) with its tiles in `cur`
    auto step = [&](const Engine32 &cur, const Engine32 &nxt, int c, bool valid) {
        const bool has_next = valid && c + 1 < c1;
        if (has_next) {
            nxt.store_q(q, (c + 1) * C, N);
            nxt.store_kv(b.k, b.v, (c + 1) * C, N);
        }
        {
            const int cn = min(c + 2, c1 - 1);
            q.template load<true>(Qh, cn * C, N, e.tid);
            b.template load<true>(Kh, Vh, cn, N, e.tid);
        }
        f32x16 Pm;
        float inv_q = 0.0f;
        if (valid) {
            const bool adv = c + 1 < c1 || advance_last;
            inv_q = __shfl(cur.row_inv<true>(), 32 * e.dh + e.l32, 64);
            Pm = cur.chunk_outputs(S, adv);
            if (adv && e.tid < 128) z += cur.z_delta();
            if (e.tid < 128) cur.set_z(z);  // for chunk c + 1
        }
        __syncthreads();  // chunk c's reads of A, the sums and its buffer done; hand-overs written
        if (valid) cur.finish(Pm, inv_q, Oh, c * C, N, poison);
        if (has_next) {
            nxt.a_tiles();
            nxt.qz_rows();
            if (c + 2 < c1 || advance_last) nxt.z_partials();
        }
        __syncthreads();
    };
    for (int c = c0; c < c1; c += 2) {
        step(e, e1, c, true);
        step(e1, e, c + 1, c + 1 < c1);
    }
}

// Phase A, decoupled look-back, phase B (as fused_causal_kernel, without the
// one-chunk shortcut: a one-chunk segment is staged twice).
template <typename OT>
__global__ __launch_bounds__(512, 1) void fused_causal32_kernel(const bf16 *__restrict__ Q, const bf16 *__restrict__ K,
                                                                const bf16 *__restrict__ V, OT *__restrict__ out,
                                                                void *ws_raw, int BH, int N, int G_, int CPS,
                                                                float *__restrict__ S_out, float *__restrict__ z_out,
                                                                const float *S_in, const float *z_in) {
    using Gc = Cfg<bf16, 128, 128, 64>;
    constexpr int C = 64, D = 128, M = 128;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Gc::bytes];
    __shared__ __attribute__((aligned(16))) float sx[8 * 4 * 64 * 4];
    __shared__ __attribute__((aligned(16))) bf16 stiles[3 * 64 * 128];  // second tile buffer
    __shared__ __attribute__((aligned(16))) float szp1[128];            // its column-sum partials (phase A)
    __shared__ unsigned sh_word[4];
    Engine32 e(smem, sx);
    Engine32 e1 = e;
    e1.sQ = stiles;
    e1.sK = stiles + 64 * 128;
    e1.sV = stiles + 2 * 64 * 128;
    e1.szp = szp1;
    const int tid = e.tid;

    // block b -> segment b / BH of head b % BH (dispatched in block order; see fused_causal_kernel)
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
    const bf16 *Qh = Q + (size_t)bh * N * D;
    const bf16 *Kh = K + (size_t)bh * N * D;
    const bf16 *Vh = V + (size_t)bh * N * M;
    OT *Oh = out + (size_t)bh * N * M;

    e.clear_a();

    f32x16 acc[2] = {zero16(), zero16()};
    float zacc = 0.0f;
    const bool last = s == G_ - 1;
    const bool want_final = S_out != nullptr;
    const bool run_a = G_ > 1 && (!last || want_final);
    if (run_a) phase_a32(e, e1, Kh, Vh, N, c0, c1, acc, zacc);
    const size_t my = (size_t)bh * G_ + s;
    f32x16 pre[2] = {zero16(), zero16()};
    float zpre = 0.0f;
    const bool init = S_in != nullptr && s == 0;
    if (init) e.state_add32(pre, zpre, S_in + (size_t)bh * D * M, z_in + (size_t)bh * D);
    f32x4 x4[8][1];
    if (G_ > 1 && !last) {
        if (init) {
            f32x16 a0[2] = {acc[0] + pre[0], acc[1] + pre[1]};
            Engine32::to4(a0, x4);
            e.slot_store(x4, zacc + zpre, ws.agg + my * Gc::EP);
        } else {
            Engine32::to4(acc, x4);
            e.slot_store(x4, zacc, ws.agg + my * Gc::EP);
        }
        e.publish_flag(&ws.flags[my], ep | 1u);
    }

    Stage<bf16, 64, 128, 512> stQ;
    stQ.template load<true>(Qh, c0 * C, N, tid);

    bool failed = false;
    if (G_ > 1 && s > 0) {
        Engine32::to4(pre, x4);
        failed = !look_back(e, ws, sh_word, bh, s, G_, ep, x4, zpre, false);
        Engine32::from4(x4, pre);
        if (!last) {
            f32x4 a4[8][1];
            Engine32::to4(acc, a4);
            publish_inclusive(e, ws, my, ep, x4, zpre, a4, zacc, failed);
        }
    }
    if (G_ > 1 && last && want_final) {
        f32x16 fin[2] = {pre[0] + acc[0], pre[1] + acc[1]};
        if (failed) {
#pragma unroll
            for (int v = 0; v < 16; ++v) fin[0][v] = fin[1][v] = __builtin_nanf("");
        }
        e.state_store32(fin, failed ? __builtin_nanf("") : zpre + zacc, S_out + (size_t)bh * D * M,
                        z_out + (size_t)bh * D);
    }

    phase_b32<OT>(e, e1, Qh, Kh, Vh, Oh, N, c0, c1, G_ == 1 && want_final, stQ, pre, zpre, failed);
    if (G_ == 1 && want_final) e.state_store32(pre, zpre, S_out + (size_t)bh * D * M, z_out + (size_t)bh * D);

    if (G_ > 1 && last) finish_call(ws, epoch, (unsigned)BH);
}

}  // namespace la
