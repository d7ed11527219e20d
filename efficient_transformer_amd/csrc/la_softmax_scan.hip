// Softmax attention of one query per head over every prefix, as an RNN.
//
// Page "Attention as an RNN" (Feng et al., 2024), Proposed method: attention is
// an RNN; its many-to-many outputs (the attention of the query over each
// prefix) follow from a running state updated token by token, and a parallel
// prefix scan computes them all at once; the query is a learned vector q.
// With s_i = q . k_i the state after position k is
//   (m_k, u_k, w_k) = (max_{i<=k} s_i, sum exp(s_i - m_k), sum exp(s_i - m_k) v_i)
// and out_k = w_k / u_k.  Two states combine associatively:
//   (m1, u1, w1) + (m2, u2, w2) = (m, u1 e^{m1-m} + u2 e^{m2-m}, w1 e^{m1-m} + w2 e^{m2-m}),
//   m = max(m1, m2).
//
// Scan kernel: one wavefront per segment of R = 32 rows of one head (lanes are
// value columns), four consecutive segments per workgroup (a group).  The
// wavefront
//   1. issues the loads of its K tile and V rows together, stages K in LDS and
//      forms s_i, one row per lane;
//   2. forms the running max, the scale factors and u_i for all rows at once
//      (shuffle scans over lanes = rows), then w_i row after row with one fma
//      per row and column, keeping every row's local state (w_i in the
//      register that held v_i; m_i, u_i in lane i);
//   3. writes its segment state to LDS; wavefront 0 combines the group's four
//      states, publishes the group state, looks back over the earlier groups of
//      the head (decoupled look-back, the same flag / epoch protocol as the
//      prefill kernels; a state is only M + 2 floats), publishes the group's
//      inclusive state and passes the prefix back through LDS; each wavefront
//      adds the states of the group's earlier segments;
//   4. writes out_i = prefix + local state of row i, normalised.
// One look-back per group of 128 rows instead of per segment: a quarter of the
// chain length and of the published states.  The last group of every head
// counts itself done after its look-back; the last head to count advances the
// epoch (as in the prefill kernels).
// Workspace: 64 header words, one flag word per group (padded to 64 words),
// then the aggregate and the inclusive state of every group (SP floats each).
#include <math.h>

#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

namespace {

constexpr long kScanSpinLimit = 1L << 22;
constexpr int kScanWaves = 4;
// With at most this many groups per head no inclusive state is published: the
// look-back reads every earlier aggregate (M + 2 floats each) in one batch,
// and wavefront 0 no longer waits for a store before writing its rows.
constexpr int kScanInclusiveMinGroups = 16;

template <int D, int M>
struct ScanCfg {
    static constexpr int R = 32;                // rows per segment (one wavefront)
    static constexpr int CPL = M > 64 ? 2 : 1;  // value columns per lane
    static constexpr int LK = D + 4;            // LDS row of the K tile (floats)
    static constexpr int SP = scan_slot_floats(M);
};

template <typename T>
__device__ __forceinline__ float ld1(const T *p) {
    return to_f32(*p);
}
template <typename T>
__device__ __forceinline__ f32x4 ld4(const T *p);
template <>
__device__ __forceinline__ f32x4 ld4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <>
__device__ __forceinline__ f32x4 ld4<bf16>(const bf16 *p) {
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

template <typename T, int D, int M>
__global__ __launch_bounds__(64 * kScanWaves) void softmax_scan_kernel(
    const T *__restrict__ q, const T *__restrict__ K, const T *__restrict__ V, float *__restrict__ out,
    void *ws_raw, int BH, int N, int NS, int NG, float *__restrict__ m_out, float *__restrict__ u_out,
    float *__restrict__ w_out) {
    using G = ScanCfg<D, M>;
    constexpr int R = G::R, CPL = G::CPL;
    __shared__ __attribute__((aligned(16))) float sk[kScanWaves][R * G::LK];
    __shared__ float sq[kScanWaves][D];
    __shared__ float sst[kScanWaves][M + 2];  // each segment's local state (w, m, u)
    __shared__ float spre[M + 3];             // the group's prefix (w, m, u) and a failure flag
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int bh = (int)(blockIdx.x % (unsigned)BH), grp = (int)(blockIdx.x / (unsigned)BH);
    const int seg = grp * kScanWaves + w;
    const int row0 = seg * R;
    const int nrows = max(0, min(R, N - row0));  // 0: a segment past the end (identity state)
    const bool last = seg == NS - 1;
    const bool last_grp = grp == NG - 1;

    unsigned *hdr = static_cast<unsigned *>(ws_raw);
    const long items = (long)BH * NG;
    unsigned *flags = hdr + kWsHeaderWords;
    float *agg = reinterpret_cast<float *>(flags + fused_flag_words(items));
    float *incl = agg + (size_t)items * G::SP;
    unsigned epoch = 0;
    if (NG > 1 && w == 0) epoch = __hip_atomic_load(&hdr[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned ep = (epoch & 0x3fffffffu) << 2;

    float wv[R][CPL];  // v_i on load, then the local w_i
    float m = -INFINITY, u = 0.0f, wl[CPL];
    float my_m = -INFINITY, my_u = 0.0f;  // lane i: the local state (m_i, u_i) of row i
#pragma unroll
    for (int c = 0; c < CPL; ++c) wl[c] = 0.0f;
    if (nrows > 0) {
        // 1. loads: the K tile (16-byte loads, staged in LDS) and the V rows (lane =
        //    column) are all issued before any of them is used; rows past N reload
        //    row nrows - 1 and are masked below.
        float *tile = sk[w];
        const T *Kh = K + ((size_t)bh * N + row0) * D;
        const T *Vh = V + ((size_t)bh * N + row0) * M;
        constexpr int KL = R * D / 4 / 64;  // 4-element K loads per lane
        f32x4 kreg[KL];
#pragma unroll
        for (int x = 0; x < KL; ++x) {
            const int e = lane + 64 * x, r = e / (D / 4), d = (e % (D / 4)) * 4;
            kreg[x] = ld4(Kh + (size_t)min(r, nrows - 1) * D + d);
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int col = min(lane + 64 * c, M - 1);
                wv[i][c] = ld1(Vh + (size_t)min(i, nrows - 1) * M + col);
            }
        for (int d = lane; d < D; d += 64) sq[w][d] = ld1(q + (size_t)bh * D + d);
#pragma unroll
        for (int x = 0; x < KL; ++x) {
            const int e = lane + 64 * x, r = e / (D / 4), d = (e % (D / 4)) * 4;
            *reinterpret_cast<f32x4 *>(tile + r * G::LK + d) = kreg[x];
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // LDS writes done (vmcnt left alone: V may be in flight)
        __builtin_amdgcn_wave_barrier();
        float s = -INFINITY;  // s of row `lane`
        if (lane < nrows) {
            float acc = 0.0f;
#pragma unroll
            for (int d4 = 0; d4 < D / 4; ++d4) {
                const f32x4 kv = *reinterpret_cast<const f32x4 *>(tile + lane * G::LK + 4 * d4);
                const f32x4 qv = *reinterpret_cast<const f32x4 *>(sq[w] + 4 * d4);
                acc += kv[0] * qv[0] + kv[1] * qv[1] + kv[2] * qv[2] + kv[3] * qv[3];
            }
            s = acc;
        }

        // 2. the segment's recurrence, with everything that does not depend on v
        //    done in parallel over rows (lane i = row i): the running max m_i (prefix
        //    max), the factors a_i = e^(m_{i-1} - m_i) and b_i = e^(s_i - m_i) of
        //    u_i = a_i u_{i-1} + b_i, and u_i itself (a scan of that affine map).
        //    Only w_i = a_i w_{i-1} + b_i v_i runs row after row, one fma per row
        //    and column.  Rows past N have s = -inf: a = 1, b = 0 keep the state.
        //    The scans over the 32 rows (lanes 0 .. 31) run on DPP moves: within each
        //    16-lane row by shifts of 1, 2, 4 and 8 lanes, then the second row takes
        //    the first row's total from its lane 15; lanes without a source lane
        //    combine with the identity.
        static_assert(R == 32, "rows are lanes 0 .. 31: two 16-lane rows");
        float mx = s;
        mx = fmaxf(mx, dpp_row_shr<1>(mx, -INFINITY));
        mx = fmaxf(mx, dpp_row_shr<2>(mx, -INFINITY));
        mx = fmaxf(mx, dpp_row_shr<4>(mx, -INFINITY));
        mx = fmaxf(mx, dpp_row_shr<8>(mx, -INFINITY));
        mx = fmaxf(mx, dpp_row_bcast15(mx, -INFINITY));
        const float mprev = dpp_wave_shr1(mx, -INFINITY);  // the running max of the rows before
        const float fa = mx == -INFINITY ? 1.0f : __expf(mprev - mx);
        const float fb = mx == -INFINITY ? 0.0f : __expf(s - mx);
        float sa = fa, su = fb;  // composition of the maps of rows <= lane: u -> sa u + su
        // after the maps of the earlier rows (pa, pb): u -> sa (pa u + pb) + su; the
        // identity (1, 0) leaves (sa, su) unchanged
        auto after = [&](float pa, float pb) {
            su = sa * pb + su;
            sa = sa * pa;
        };
        after(dpp_row_shr<1>(sa, 1.0f), dpp_row_shr<1>(su, 0.0f));
        after(dpp_row_shr<2>(sa, 1.0f), dpp_row_shr<2>(su, 0.0f));
        after(dpp_row_shr<4>(sa, 1.0f), dpp_row_shr<4>(su, 0.0f));
        after(dpp_row_shr<8>(sa, 1.0f), dpp_row_shr<8>(su, 0.0f));
        after(dpp_row_bcast15(sa, 1.0f), dpp_row_bcast15(su, 0.0f));
        my_m = mx;
        my_u = su;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float ai = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fa), i));
            const float bi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fb), i));
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                wl[c] = __builtin_fmaf(wl[c], ai, bi * wv[i][c]);
                wv[i][c] = wl[c];
            }
        }
        m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), R - 1));
        u = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, su), R - 1));
    }

    // (pm, pu, pw) = (pm, pu, pw) + (sm, su, sw): the state comes after the prefix
    float pm = -INFINITY, pu = 0.0f, pw[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) pw[c] = 0.0f;
    auto add_back = [&](float sm, float sus, const float *sw) {
        if (sm != sm) {
            // a state published by a group whose wait gave up (its max is NaN):
            // the prefix is lost.  fmaxf would drop the NaN (and an empty prefix
            // would then skip the state), so the loss is made explicit here; the
            // NaN sums stay NaN through every later combination.
            pm = __builtin_nanf("");
            pu = __builtin_nanf("");
#pragma unroll
            for (int c = 0; c < CPL; ++c) pw[c] = __builtin_nanf("");
            return;
        }
        const float mn = fmaxf(sm, pm);
        if (mn != -INFINITY) {
            const float a = __expf(pm - mn), b = __expf(sm - mn);
            pu = pu * a + sus * b;
#pragma unroll
            for (int c = 0; c < CPL; ++c) pw[c] = pw[c] * a + sw[c] * b;
            pm = mn;
        }
    };

    // 3. the segments of the group exchange their states through LDS; one
    //    wavefront publishes the group's state and looks back over the earlier
    //    groups of the head (decoupled look-back); the prefix comes back through LDS.
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        if (lane + 64 * c < M) sst[w][lane + 64 * c] = wl[c];
    if (lane == 0) {
        sst[w][M] = m;
        sst[w][M + 1] = u;
    }
    __syncthreads();
    auto add_lds = [&](const float *st) {
        float sw[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) sw[c] = lane + 64 * c < M ? st[lane + 64 * c] : 0.0f;
        add_back(st[M], st[M + 1], sw);
    };
    bool failed = false;
    const size_t my = (size_t)grp * BH + bh;  // item of this group
    auto store_state = [&](float *slot, float sm, float sus, const float *sw) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int col = lane + 64 * c;
            if (col < M) __hip_atomic_store(slot + col, sw[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) {
            __hip_atomic_store(slot + M, sm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(slot + M + 1, sus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    auto publish = [&](unsigned value) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(&flags[my], value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    float gm = -INFINITY, gu = 0.0f, gw[CPL];  // wavefront 0: the group's aggregate
#pragma unroll
    for (int c = 0; c < CPL; ++c) gw[c] = 0.0f;
    if (NG > 1 && w == 0) {
        // the group's aggregate: its segments in order
        for (int k = 0; k < kScanWaves; ++k) add_lds(sst[k]);
        gm = pm;
        gu = pu;
#pragma unroll
        for (int c = 0; c < CPL; ++c) gw[c] = pw[c];
        if (!last_grp) {
            store_state(agg + my * G::SP, gm, gu, gw);
            publish(ep | 1u);
        }
        pm = -INFINITY;
        pu = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) pw[c] = 0.0f;
        if (grp > 0) {
            // load up to LB states at once (their latencies overlap), then combine in order
            constexpr int LB = 16;
            auto add_slots = [&](const float *first, int j0, int j1) {  // first, then agg of groups j0 .. j1-1
                {
                    float sw[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) sw[c] = lane + 64 * c < M ? first[lane + 64 * c] : 0.0f;
                    add_back(first[M], first[M + 1], sw);
                }
                for (int jb = j0; jb < j1; jb += LB) {
                    float tm[LB], tu[LB], tw[LB][CPL];
#pragma unroll
                    for (int k = 0; k < LB; ++k) {
                        const int j = jb + k < j1 ? jb + k : jb;
                        const float *slot = agg + ((size_t)j * BH + bh) * G::SP;
                        tm[k] = slot[M];
                        tu[k] = slot[M + 1];
#pragma unroll
                        for (int c = 0; c < CPL; ++c) tw[k][c] = lane + 64 * c < M ? slot[lane + 64 * c] : 0.0f;
                    }
#pragma unroll
                    for (int k = 0; k < LB; ++k)
                        if (jb + k < j1) add_back(tm[k], tu[k], tw[k]);
                }
            };
            int base = grp - 1;
            int jstar = -1;
            long spins = 0;
            // header word 4, when the host has set it, caps the polls (tests of the give-up path)
            const unsigned cap = __hip_atomic_load(&hdr[kWsPollCapWord], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const long limit = cap != 0u ? (long)cap : kScanSpinLimit;
            while (true) {
                const int j = base - lane;
                unsigned f = 0u;
                if (j >= 0)
                    f = __hip_atomic_load(flags + (size_t)j * BH + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const bool ok = j >= 0 && (f & ~3u) == ep && (f & 3u) != 0u;
                const bool inc = ok && ((f & 3u) == 2u || j == 0);
                const unsigned long long okm = __ballot(ok), incm = __ballot(inc);
                if (incm != 0ull) {
                    const int first = __builtin_ctzll(incm);
                    const unsigned long long need = first == 63 ? ~0ull : ((1ull << (first + 1)) - 1ull);
                    if ((okm & need) == need) {
                        jstar = base - first;
                        break;
                    }
                } else if (okm == ~0ull) {
                    base -= 64;
                    continue;
                }
                if (++spins > limit) {
                    if (lane == 0) __hip_atomic_store(&hdr[kWsErrorWord], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (jstar < 0) {
                failed = true;
            } else {
                add_slots((jstar == 0 ? agg : incl) + ((size_t)jstar * BH + bh) * G::SP, jstar + 1, grp);
            }
        }
        if (last_grp && lane == 0) {
            // every group of this head has read the epoch (see the prefill kernels'
            // finish_call): count the head, and the last head advances the epoch
            const unsigned done = atomicAdd(&hdr[1], 1u);
            if (done == (unsigned)BH - 1u) {
                __hip_atomic_store(&hdr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&hdr[2], epoch + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            if (lane + 64 * c < M) spre[lane + 64 * c] = pw[c];
        if (lane == 0) {
            spre[M] = pm;
            spre[M + 1] = pu;
            spre[M + 2] = failed ? 1.0f : 0.0f;
        }
    }
    if (NG > 1) {
        __syncthreads();
        pm = -INFINITY;
        pu = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) pw[c] = 0.0f;
        add_lds(spre);
        failed = spre[M + 2] != 0.0f;
        if (w == 0 && grp > 0 && !last_grp && NG > kScanInclusiveMinGroups) {
            // the group's inclusive state = prefix + aggregate, published once the
            // other wavefronts have their prefix (later groups can use aggregates)
            const float mn = fmaxf(pm, gm);
            const float a = mn == -INFINITY ? 0.0f : __expf(pm - mn), b = mn == -INFINITY ? 0.0f : __expf(gm - mn);
            float iw[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) iw[c] = failed ? __builtin_nanf("") : pw[c] * a + gw[c] * b;
            store_state(incl + my * G::SP, failed ? __builtin_nanf("") : mn, pu * a + gu * b, iw);
            publish(ep | 2u);
        }
    }
    // the earlier segments of this group follow the group's prefix
    for (int k = 0; k < w; ++k) add_lds(sst[k]);

    if (last && m_out != nullptr) {
        const float mn = fmaxf(pm, m);
        const float a = mn == -INFINITY ? 0.0f : __expf(pm - mn), b = mn == -INFINITY ? 0.0f : __expf(m - mn);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int col = lane + 64 * c;
            if (col < M) w_out[(size_t)bh * M + col] = failed ? __builtin_nanf("") : pw[c] * a + wl[c] * b;
        }
        if (lane == 0) {
            m_out[bh] = failed ? __builtin_nanf("") : mn;
            u_out[bh] = failed ? __builtin_nanf("") : pu * a + u * b;
        }
    }

    // 4. outputs: row i = prefix + local state of row i, normalised; the factors of
    //    row i are formed in lane i, then each row is one fma per column
    if (nrows > 0) {
        float *Oh = out + ((size_t)bh * N + row0) * M;
        const float mxp = fmaxf(pm, my_m);
        const float al = mxp == -INFINITY ? 0.0f : __expf(pm - mxp);  // pm = -inf: 0
        const float be = mxp == -INFINITY ? 0.0f : __expf(my_m - mxp);
        const float inv = 1.0f / (pu * al + my_u * be);
        const float oa = failed ? __builtin_nanf("") : al * inv, ob = be * inv;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            if (i >= nrows) break;
            const float ai = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, oa), i));
            const float bi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ob), i));
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int col = lane + 64 * c;
                if (col < M) Oh[(size_t)i * M + col] = __builtin_fmaf(pw[c], ai, wv[i][c] * bi);
            }
        }
    }
}

// One token of the RNN for every head: one wavefront per head, lanes = value
// columns; s = q . k reduced over the wavefront.
template <typename T, int D, int M>
__global__ __launch_bounds__(64) void softmax_step_kernel(float *__restrict__ m, float *__restrict__ u,
                                                          float *__restrict__ w, const T *__restrict__ q,
                                                          const T *__restrict__ k, const T *__restrict__ v,
                                                          float *__restrict__ out) {
    constexpr int CPL = M > 64 ? 2 : 1;
    const int lane = threadIdx.x;
    const size_t h = blockIdx.x;
    float s = 0.0f;
    for (int d = lane; d < D; d += 64) s += ld1(q + h * D + d) * ld1(k + h * D + d);
    s = row_group_sum<16>(s);
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    const float m0 = m[h], u0 = u[h];
    const float mn = fmaxf(m0, s);
    const float a = __expf(m0 - mn), b = __expf(s - mn);
    const float un = u0 * a + b;
    const float inv = 1.0f / un;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int col = lane + 64 * c;
        if (col < M) {
            const float wn = w[h * M + col] * a + b * ld1(v + h * M + col);
            w[h * M + col] = wn;
            out[h * M + col] = wn * inv;
        }
    }
    if (lane == 0) {
        m[h] = mn;
        u[h] = un;
    }
}

template <typename T, int D, int M>
hipError_t run_scan(const void *q, const void *K, const void *V, float *out, void *ws, int BH, int N, float *m_out,
                    float *u_out, float *w_out, hipStream_t stream) {
    const int NS = (N + ScanCfg<D, M>::R - 1) / ScanCfg<D, M>::R;
    const int NG = (NS + kScanWaves - 1) / kScanWaves;
    const long groups = (long)BH * NG;
    if (groups <= 0) return hipSuccess;
    hipLaunchKernelGGL((softmax_scan_kernel<T, D, M>), dim3((unsigned)groups), dim3(64 * kScanWaves), 0, stream,
                       (const T *)q, (const T *)K, (const T *)V, out, ws, BH, N, NS, NG, m_out, u_out, w_out);
    return hipGetLastError();
}

template <typename T, int D, int M>
hipError_t run_step(float *m, float *u, float *w, const void *q, const void *k, const void *v, float *out, int BH,
                    hipStream_t stream) {
    if (BH <= 0) return hipSuccess;
    hipLaunchKernelGGL((softmax_step_kernel<T, D, M>), dim3((unsigned)BH), dim3(64), 0, stream, m, u, w,
                       (const T *)q, (const T *)k, (const T *)v, out);
    return hipGetLastError();
}

}  // namespace

int softmax_scan_rows(int) { return 32 * kScanWaves; }  // rows per group (one look-back each)

hipError_t softmax_scan(int dtype, int D, int M, const void *q, const void *K, const void *V, float *out, void *ws,
                        int BH, int N, float *m_out, float *u_out, float *w_out, hipStream_t stream) {
#define X(D_, M_)                                                                                              \
    if (D == D_ && M == M_)                                                                                    \
        return dtype == 0 ? run_scan<float, D_, M_>(q, K, V, out, ws, BH, N, m_out, u_out, w_out, stream)    \
                          : run_scan<bf16, D_, M_>(q, K, V, out, ws, BH, N, m_out, u_out, w_out, stream);
#define XM(D_) X(D_, 16) X(D_, 32) X(D_, 64) X(D_, 128)
    XM(16) XM(32) XM(64) XM(128)
#undef XM
#undef X
    return hipErrorInvalidValue;
}

hipError_t softmax_step(int dtype, int D, int M, float *m, float *u, float *w, const void *q, const void *k,
                        const void *v, float *out, int BH, hipStream_t stream) {
#define X(D_, M_)                                                                              \
    if (D == D_ && M == M_)                                                                    \
        return dtype == 0 ? run_step<float, D_, M_>(m, u, w, q, k, v, out, BH, stream)         \
                          : run_step<bf16, D_, M_>(m, u, w, q, k, v, out, BH, stream);
#define XM(D_) X(D_, 16) X(D_, 32) X(D_, 64) X(D_, 128)
    XM(16) XM(32) XM(64) XM(128)
#undef XM
#undef X
    return hipErrorInvalidValue;
}

}  // namespace la
