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
// value columns).  The wavefront
//   1. stages its K tile in LDS (coalesced) and forms s_i, one row per lane;
//   2. runs the recurrence over its rows, keeping every row's local state
//      (w_i in the register that held v_i; m_i, u_i in lane i);
//   3. publishes its segment state, looks back over the earlier segments of the
//      head (decoupled look-back, the same flag / epoch protocol as the prefill
//      kernels; a state is only M + 2 floats) and publishes its inclusive state;
//   4. writes out_i = prefix + local state of row i, normalised.
// The last segment of every head counts itself done after its look-back; the
// last head to count advances the epoch (as in the prefill kernels).
// Workspace: 64 header words, one flag word per segment (padded to 64 words),
// then the aggregate and the inclusive state of every segment (SP floats each).
#include <math.h>

#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

namespace {

constexpr long kScanSpinLimit = 1L << 22;
constexpr int kScanWaves = 4;

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

template <typename T, int D, int M>
__global__ __launch_bounds__(64 * kScanWaves) void softmax_scan_kernel(
    const T *__restrict__ q, const T *__restrict__ K, const T *__restrict__ V, float *__restrict__ out,
    void *ws_raw, int BH, int N, int NS, float *__restrict__ m_out, float *__restrict__ u_out,
    float *__restrict__ w_out) {
    using G = ScanCfg<D, M>;
    constexpr int R = G::R, CPL = G::CPL;
    __shared__ __attribute__((aligned(16))) float sk[kScanWaves][R * G::LK];
    __shared__ float sq[kScanWaves][D];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const long items = (long)BH * NS;
    const long gi = (long)blockIdx.x * kScanWaves + w;
    if (gi >= items) return;  // whole wavefronts only; no workgroup barrier below
    const int bh = (int)(gi % BH), seg = (int)(gi / BH);
    const int row0 = seg * R;
    const int nrows = min(R, N - row0);
    const bool last = seg == NS - 1;

    unsigned *hdr = static_cast<unsigned *>(ws_raw);
    unsigned *flags = hdr + kWsHeaderWords;
    float *agg = reinterpret_cast<float *>(flags + fused_flag_words(items));
    float *incl = agg + (size_t)items * G::SP;
    unsigned epoch = 0;
    if (NS > 1) epoch = __hip_atomic_load(&hdr[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned ep = (epoch & 0x3fffffffu) << 2;

    // 1. scores: K tile through LDS (rows past N are zero), q in LDS
    float *tile = sk[w];
    const T *Kh = K + ((size_t)bh * N + row0) * D;
    for (int x = lane; x < R * D; x += 64) {
        const int r = x / D, d = x % D;
        tile[r * G::LK + d] = r < nrows ? ld1(Kh + (size_t)r * D + d) : 0.0f;
    }
    for (int d = lane; d < D; d += 64) sq[w][d] = ld1(q + (size_t)bh * D + d);
    __builtin_amdgcn_s_waitcnt(0);
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

    // 2. local recurrence over the segment's rows; lanes = value columns
    const T *Vh = V + ((size_t)bh * N + row0) * M;
    float wv[R][CPL];  // v_i on load, then the local w_i
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int col = lane + 64 * c;
            wv[i][c] = (col < M && i < nrows) ? ld1(Vh + (size_t)i * M + col) : 0.0f;
        }
    float m = -INFINITY, u = 0.0f;
    float wl[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) wl[c] = 0.0f;
    float my_m = -INFINITY, my_u = 0.0f;  // lane i: the local state of row i
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const float si = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), i));
        if (si != -INFINITY) {  // uniform: rows past N leave the state as it is
            const float mn = fmaxf(m, si);
            const float a = __expf(m - mn), b = __expf(si - mn);
            u = u * a + b;
#pragma unroll
            for (int c = 0; c < CPL; ++c) wl[c] = wl[c] * a + b * wv[i][c];
            m = mn;
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) wv[i][c] = wl[c];
        if (lane == i) {
            my_m = m;
            my_u = u;
        }
    }

    // 3. publish the segment state; look back for the prefix
    const size_t my = (size_t)gi;
    float pm = -INFINITY, pu = 0.0f, pw[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) pw[c] = 0.0f;
    bool failed = false;
    auto store_state = [&](float *slot, float sm, float su, const float *sw) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int col = lane + 64 * c;
            if (col < M) __hip_atomic_store(slot + col, sw[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) {
            __hip_atomic_store(slot + M, sm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(slot + M + 1, su, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    auto publish = [&](unsigned value) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(&flags[my], value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // prefix (pm, pu, pw) = prefix + state (sm, su, sw): the state comes after the prefix
    auto add_back = [&](float sm, float su, const float *sw) {
        const float mn = fmaxf(sm, pm);
        if (mn != -INFINITY) {
            const float a = __expf(pm - mn), b = __expf(sm - mn);
            pu = pu * a + su * b;
#pragma unroll
            for (int c = 0; c < CPL; ++c) pw[c] = pw[c] * a + sw[c] * b;
            pm = mn;
        }
    };
    // load up to LB states at once (their latencies overlap), then combine in order
    constexpr int LB = 16;
    auto add_slots = [&](const float *first, int j0, int j1) {  // first, then agg of segments j0 .. j1-1
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
    if (NS > 1 && !last) {
        store_state(agg + my * G::SP, m, u, wl);
        publish(ep | 1u);
    }
    if (NS > 1 && seg > 0) {
        const unsigned *fl = flags;  // flag of segment j of this head: item j * BH + bh
        int base = seg - 1;
        int jstar = -1;
        long spins = 0;
        while (true) {
            const int j = base - lane;
            unsigned f = 0u;
            if (j >= 0) f = __hip_atomic_load(fl + (size_t)j * BH + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
            if (++spins > kScanSpinLimit) {
                if (lane == 0) __hip_atomic_store(&hdr[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (jstar < 0) {
            failed = true;
        } else {
            add_slots((jstar == 0 ? agg : incl) + ((size_t)jstar * BH + bh) * G::SP, jstar + 1, seg);
        }
        if (!last) {
            // inclusive = prefix + local
            const float mn = fmaxf(pm, m);
            const float a = __expf(pm - mn), b = __expf(m - mn);
            float iw[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) iw[c] = failed ? __builtin_nanf("") : pw[c] * a + wl[c] * b;
            store_state(incl + my * G::SP, failed ? __builtin_nanf("") : mn, pu * a + u * b, iw);
            publish(ep | 2u);
        }
    }
    if (NS > 1 && last && lane == 0) {
        // every segment of this head has read the epoch (see the prefill kernels'
        // finish_call): count the head, and the last head advances the epoch
        const unsigned done = atomicAdd(&hdr[1], 1u);
        if (done == (unsigned)BH - 1u) {
            __hip_atomic_store(&hdr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hdr[2], epoch + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (last && m_out != nullptr) {
        const float mn = fmaxf(pm, m);
        const float a = mn == -INFINITY ? 0.0f : __expf(pm - mn), b = mn == -INFINITY ? 0.0f : __expf(m - mn);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int col = lane + 64 * c;
            if (col < M) w_out[(size_t)bh * M + col] = pw[c] * a + wl[c] * b;
        }
        if (lane == 0) {
            m_out[bh] = mn;
            u_out[bh] = pu * a + u * b;
        }
    }

    // 4. outputs: row i = prefix + local state of row i, normalised
    float *Oh = out + ((size_t)bh * N + row0) * M;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        if (i >= nrows) break;
        const float mi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_m), i));
        const float ui = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_u), i));
        const float mn = fmaxf(pm, mi);
        const float a = __expf(pm - mn), b = __expf(mi - mn);  // pm = -inf: a = 0
        const float inv = 1.0f / (pu * a + ui * b);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int col = lane + 64 * c;
            if (col < M) Oh[(size_t)i * M + col] = failed ? __builtin_nanf("") : (pw[c] * a + wv[i][c] * b) * inv;
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
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
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
    const long items = (long)BH * NS;
    if (items <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((items + kScanWaves - 1) / kScanWaves);
    hipLaunchKernelGGL((softmax_scan_kernel<T, D, M>), dim3(blocks), dim3(64 * kScanWaves), 0, stream, (const T *)q,
                       (const T *)K, (const T *)V, out, ws, BH, N, NS, m_out, u_out, w_out);
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

int softmax_scan_rows(int) { return 32; }

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
