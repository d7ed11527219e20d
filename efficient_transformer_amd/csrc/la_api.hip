// C ABI of the linear-attention library: argument validation, planning, launch.
// Declarations and the contract of every entry point are in include/linattn.h.
#include <limits.h>

#include <algorithm>
#include <mutex>

#include "la_launch.hpp"
#include "linattn.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

// la_decode_steps: the chunked kernels beat the register recurrence from about
// 12 tokens per head for states of 4096+ values, 16 tokens for 2048+, 32 for any
// (crossovers measured on MI355X with 2048 heads).
bool decode_steps_chunked(int64_t T, int64_t D, int64_t M) {
    return (T >= 12 && D * M >= 4096) || (T >= 16 && D * M >= 2048) || T >= 32;
}

// widths with specialised kernels
bool dim_ok(int64_t x) { return x == 16 || x == 32 || x == 64 || x == 128; }
// widths the prefill and decode entry points also take: multiples of 16 up to
// 128; those without a kernel of their own run on tiles of the next width up
bool dim_padded_ok(int64_t x) { return x >= 16 && x <= 128 && x % 16 == 0; }
int64_t dim_up(int64_t x) { return x <= 16 ? 16 : x <= 32 ? 32 : x <= 64 ? 64 : 128; }
size_t round256(size_t x) { return (x + 255) / 256 * 256; }
// B * H > lim, for B, H >= 0, without forming a product that can overflow
bool bh_over(int64_t B, int64_t H, int64_t lim) { return B > lim || H > lim || (B > 0 && H > lim / B); }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

struct Plan {
    int chunk = 0;
    int segments = 0;
    int chunks_per_segment = 0;
    int nstates = 0;  // segment states the causal/non-causal path computes
    bool onepass = false;  // causal: one-pass kernel (segments of at most 4 chunks)
    size_t ws_bytes = 0;
    // D or M without a kernel of its own: the kernels run at widths Dk, Mk on
    // padded copies held in the workspace after the kernels' own inner_ws bytes
    bool padded = false;
    int64_t Dk = 0, Mk = 0;
    size_t inner_ws = 0, oQ = 0, oK = 0, oV = 0, oO = 0, oS = 0, oZ = 0;
    // la_forward_features in two launches (map, then attention on the features held
    // in the workspace at oQ, oK; bf16 V widened to fp32 at oV): the attention's plan
    bool split = false;
    int att_chunk = 0, att_segments = 0, att_cps = 0;
    bool att_onepass = false;
};

// Validate the shape arguments shared by the prefill entry points.
int check_shape(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype, bool allow_pad = false) {
    if (B < 0 || H < 0 || N < 0 || D <= 0 || M <= 0) return LA_ERR_INVALID_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16 && dtype != LA_F32_FEATURES && dtype != (LA_BF16 | LA_OUT_BF16))
        return LA_ERR_INVALID_ARG;
    if (!dim_ok(D) || !dim_ok(M)) {
        if (!allow_pad || !dim_padded_ok(D) || !dim_padded_ok(M)) return LA_ERR_UNSUPPORTED;
    }
    // index arithmetic uses int for counts and size_t for element offsets
    if (N > INT_MAX || bh_over(B, H, INT_MAX / 8)) return LA_ERR_UNSUPPORTED;
    if (B > 0 && H > 0 && N > 0) {
        const int64_t per_head = N * (D > M ? D : M);
        if (per_head > INT64_MAX / (B * H)) return LA_ERR_UNSUPPORTED;
    }
    return LA_OK;
}

size_t state_ws_bytes(int64_t BH, int64_t D, int64_t M, int G) {
    return (size_t)BH * (size_t)(G + 1) * (size_t)(D * M + D) * sizeof(float);
}

// The planner: chunk length, number of segments and workspace.
int make_plan(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal, int dtype, int chunk_req,
              Plan *plan, int64_t target_wg_override = 0, bool allow_pad = false) {
    int st = check_shape(B, H, N, D, M, dtype, allow_pad);
    if (st != LA_OK) return st;
    if (!dim_ok(D) || !dim_ok(M)) {
        // the kernels' plan at the padded widths, then room for the padded copies
        const int64_t Dk = dim_up(D), Mk = dim_up(M);
        st = make_plan(B, H, N, Dk, Mk, causal, dtype, chunk_req, plan, target_wg_override, false);
        if (st != LA_OK) return st;
        plan->padded = true;
        plan->Dk = Dk;
        plan->Mk = Mk;
        const int64_t BH = B * H;
        if (BH == 0 || N == 0) return LA_OK;
        if (BH * N > INT64_MAX / 1024) return LA_ERR_UNSUPPORTED;
        const size_t s_in = (dtype & ~LA_OUT_BF16) == LA_BF16 ? 2 : 4, s_out = (dtype & LA_OUT_BF16) ? 2 : 4;
        const size_t rows = (size_t)BH * (size_t)N;
        plan->inner_ws = plan->ws_bytes;
        // at least one 256-byte block in front: its header words stay zero when the
        // kernels need no workspace, so la_workspace_status reads a clean error word
        size_t off = round256(plan->ws_bytes > 256 ? plan->ws_bytes : 256);
        plan->oQ = off;
        off += round256(rows * Dk * s_in);
        plan->oK = off;
        off += round256(rows * Dk * s_in);
        plan->oV = off;
        off += round256(rows * Mk * s_in);
        plan->oO = off;
        off += round256(rows * Mk * s_out);
        plan->oS = off;
        off += round256((size_t)BH * Dk * Mk * 4);
        plan->oZ = off;
        off += round256((size_t)BH * Dk * 4);
        plan->ws_bytes = off;
        return LA_OK;
    }
    if (causal != 0 && causal != 1) return LA_ERR_INVALID_ARG;
    int C = 0;
    if (chunk_req == 0) {
        // fp32 operands with a small state run 32-position chunks (less masked
        // quadratic work per position on the slower fp32 MFMA); otherwise 64
        C = ((dtype & ~LA_OUT_BF16) != LA_BF16 && D * M <= 4096) ? 32 : 64;
        if (!la::prefill_supported(dtype, (int)D, (int)M, C)) C = 32;
        if (!la::prefill_supported(dtype, (int)D, (int)M, C)) C = 16;
    } else if (chunk_req == 16 || chunk_req == 32 || chunk_req == 64) {
        C = chunk_req;
    } else {
        return LA_ERR_UNSUPPORTED;
    }
    if (C == 0 || !la::prefill_supported(dtype, (int)D, (int)M, C)) return LA_ERR_UNSUPPORTED;
    plan->chunk = C;
    const int64_t BH = B * H;
    if (BH == 0 || N == 0) {
        plan->segments = 0;
        plan->chunks_per_segment = 0;
        plan->nstates = 0;
        plan->ws_bytes = 0;
        return LA_OK;
    }
    const int64_t n_chunks = (N + C - 1) / C;
    // One workgroup per segment; all workgroups of a call resident at once: 256
    // compute units times the workgroups that fit on one (four when the state is
    // at most 1024 values, two up to 64 x 64, one otherwise).  Segments are whole
    // chunks; every segment carries (D*M + D) floats of published state, so
    // fewer, longer segments.  (16 features x 64 values, headline shape: 512
    // workgroups 22.4 us, 1024 workgroups 19.8 us.)
    // Causal: the fused kernel (look-back across segments).
    // Non-causal: the three stage kernels, with segments sized the same way.
    const int64_t target_wg = target_wg_override > 0 ? target_wg_override
                              : (D * M <= 1024) ? 1024 : (D * M <= 4096) ? 512 : 256;
    int64_t cps = (n_chunks * BH + target_wg - 1) / target_wg;
    if (cps < 1) cps = 1;
    // a causal head of at most kOnePassMaxChunks chunks stays one segment: splitting
    // it only adds a look-back chain to a launch-bound call (64 positions at chunk
    // 16: 12.4 -> 9.5 us per call with one segment instead of four)
    if (causal && n_chunks <= la::kOnePassMaxChunks) cps = n_chunks;
    int64_t G = (n_chunks + cps - 1) / cps;
    cps = (n_chunks + G - 1) / G;
    G = (n_chunks + cps - 1) / cps;
    if (BH * G > INT_MAX / 256) return LA_ERR_UNSUPPORTED;
    plan->segments = (int)G;
    plan->chunks_per_segment = (int)cps;
    const int E = (int)(D * M + D);
    if (causal) {
        plan->nstates = 0;
        plan->onepass = cps <= la::kOnePassMaxChunks && la::prefill_onepass_supported(dtype, (int)D, (int)M, C);
        plan->ws_bytes = G == 1 ? 0 : la::fused_ws_bytes(BH, (int)G, E);
    } else {
        plan->nstates = (int)G;
        plan->ws_bytes = state_ws_bytes(BH, D, M, (int)G);
    }
    return LA_OK;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_HIP; }

// A padded plan (Plan::padded): copy Q and K into rows Dk wide (extra columns
// -inf, which phi maps to exactly 0; 0 for inputs that already hold features),
// V into rows Mk wide (extra columns 0) and a carried state into [Dk][Mk] (zeros
// outside), run the kernels of the plan on those, then copy the first M columns
// of every output row and the [D][M] corner of the final state back.
hipError_t run_padded(const Plan &p, const void *Q, const void *K, const void *V, void *out, int64_t BH, int64_t N,
                      int64_t D, int64_t M, int causal, int dtype, void *workspace, const float *S_in,
                      const float *z_in, float *S_out, float *z_out, hipStream_t s) {
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const long Dk = (long)p.Dk, Mk = (long)p.Mk;
    const int base = dtype & ~LA_OUT_BF16;
    const long s_in = base == LA_BF16 ? 2 : 4, s_out = (dtype & LA_OUT_BF16) ? 2 : 4;
    const unsigned fill = base == LA_F32_FEATURES ? 0u : base == LA_BF16 ? 0xFF80FF80u : 0xFF800000u;
    void *Qp = ws + p.oQ, *Kp = ws + p.oK, *Vp = ws + p.oV, *Op = ws + p.oO;
    float *Sp = reinterpret_cast<float *>(ws + p.oS), *zp = reinterpret_cast<float *>(ws + p.oZ);
    hipError_t e = la::pad_copy(Q, Qp, BH, N, D * s_in, N, Dk * s_in, fill, s);
    if (e == hipSuccess) e = la::pad_copy(K, Kp, BH, N, D * s_in, N, Dk * s_in, fill, s);
    if (e == hipSuccess) e = la::pad_copy(V, Vp, BH, N, M * s_in, N, Mk * s_in, 0u, s);
    if (e == hipSuccess && S_in) {
        e = la::pad_copy(S_in, Sp, BH, D, M * 4, Dk, Mk * 4, 0u, s);
        if (e == hipSuccess) e = la::pad_copy(z_in, zp, BH, 1, D * 4, 1, Dk * 4, 0u, s);
    }
    float *So = S_out ? Sp : nullptr, *zo = S_out ? zp : nullptr;
    const float *Si = S_in ? Sp : nullptr, *zi = S_in ? zp : nullptr;
    void *iw = p.inner_ws > 0 ? workspace : nullptr;
    const int Di = (int)Dk, Mi = (int)Mk, C = p.chunk, G = p.segments, cps = p.chunks_per_segment;
    const int bh = (int)BH, n = (int)N;
    if (e == hipSuccess) {
        if (causal && p.onepass) {
            e = la::prefill_onepass(dtype, Di, Mi, C, Qp, Kp, Vp, Op, iw, bh, n, G, cps, So, zo, Si, zi, s);
        } else if (causal) {
            e = la::prefill_fused(dtype, Di, Mi, C, Qp, Kp, Vp, Op, iw, bh, n, G, cps, So, zo, Si, zi, s);
        } else {
            float *sw = static_cast<float *>(iw);
            e = la::prefill_states(dtype, Di, Mi, C, Kp, Vp, sw, bh, n, G, cps, G, s);
            if (e == hipSuccess) e = la::prefill_scan(sw, bh, Di, Mi, G, G, So, zo, s);
            if (e == hipSuccess)
                e = la::prefill_outputs(dtype, Di, Mi, C, Qp, Kp, Vp, Op, sw, bh, n, G, cps, 0, nullptr, nullptr, s);
        }
    }
    if (e == hipSuccess) e = la::unpad_copy(Op, out, BH, N, M * s_out, N, Mk * s_out, s);
    if (e == hipSuccess && S_out) {
        e = la::unpad_copy(Sp, S_out, BH, D, M * 4, Dk, Mk * 4, s);
        if (e == hipSuccess) e = la::unpad_copy(zp, z_out, BH, 1, D * 4, 1, Dk * 4, s);
    }
    return e;
}

// ---- scratch of la_forward_chunked_noalloc ----------------------------------
// A file-scope device array (each device that loads the library holds its own
// copy until the process ends).  Host code never passes `scratch` itself to a
// kernel: its name on the host is a stand-in, not a device address.  The
// address on each device comes from hipGetSymbolAddress, taken once per device
// with that device current, and is kept in scratch_ptr.
constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device, or nullptr when it cannot be had.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

LA_API const char *la_status_str(int status) {
    switch (status) {
        case LA_OK: return "LA_OK";
        case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG: invalid argument";
        case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: unsupported shape, chunk or plan";
        case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or too small";
        case LA_ERR_HIP: return "LA_ERR_HIP: HIP runtime error at launch";
        case LA_ERR_GAVE_UP:
            return "LA_ERR_GAVE_UP: a wait for earlier segments gave up; the calls' outputs hold NaN rows";
        default: return "unknown status";
    }
}

LA_API int la_version(void) { return kVersion; }

LA_API int la_forward_plan(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal, int dtype,
                           int chunk_req, int *chunk_out, int *segments_out, size_t *workspace_bytes_out) {
    Plan p;
    const int st = make_plan(B, H, N, D, M, causal, dtype, chunk_req, &p, 0, true);
    if (st != LA_OK) return st;
    if (chunk_out) *chunk_out = p.chunk;
    if (segments_out) *segments_out = p.segments;
    if (workspace_bytes_out) *workspace_bytes_out = p.ws_bytes;
    return LA_OK;
}

LA_API size_t la_forward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal,
                                         int dtype, int chunk_req) {
    Plan p;
    return make_plan(B, H, N, D, M, causal, dtype, chunk_req, &p, 0, true) == LA_OK ? p.ws_bytes : 0;
}

LA_API int la_forward_chunked(const void *Q, const void *K, const void *V, void *out, int64_t B, int64_t H,
                              int64_t N, int64_t D, int64_t M, int causal, int dtype, int chunk_req,
                              void *workspace, size_t workspace_bytes, float *S_out, float *z_out, void *stream) {
    Plan p;
    int st = make_plan(B, H, N, D, M, causal, dtype, chunk_req, &p, 0, true);
    if (st != LA_OK) return st;
    if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_INVALID_ARG;
    if (S_out && (!aligned16(S_out) || !aligned16(z_out))) return LA_ERR_INVALID_ARG;
    const int64_t BH = B * H;
    if (BH == 0) return LA_OK;
    hipStream_t s = as_stream(stream);
    if (N == 0) {
        if (S_out == nullptr) return LA_OK;
        hipError_t e = la::fill_zero(S_out, (size_t)(BH * D * M), s);
        if (e == hipSuccess) e = la::fill_zero(z_out, (size_t)(BH * D), s);
        return hip_status(e);
    }
    if (!Q || !K || !V || !out) return LA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(out)) return LA_ERR_INVALID_ARG;
    if (p.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < p.ws_bytes)) return LA_ERR_WORKSPACE;
    if (p.ws_bytes > 0 && !aligned16(workspace)) return LA_ERR_INVALID_ARG;
    const int dt = dtype, Di = (int)D, Mi = (int)M, C = p.chunk, G = p.segments, cps = p.chunks_per_segment;
    (void)hipGetLastError();  // clear a stale error so that the checks below report this call's launches
    if (p.padded)
        return hip_status(run_padded(p, Q, K, V, out, BH, N, D, M, causal, dtype, workspace, nullptr, nullptr, S_out,
                                     z_out, s));
    hipError_t e = hipSuccess;
    if (causal && p.onepass) {
        e = la::prefill_onepass(dt, Di, Mi, C, Q, K, V, out, workspace, (int)BH, (int)N, G, cps, S_out, z_out,
                                nullptr, nullptr, s);
    } else if (causal) {
        e = la::prefill_fused(dt, Di, Mi, C, Q, K, V, out, workspace, (int)BH, (int)N, G, cps, S_out, z_out, nullptr,
                              nullptr, s);
    } else {
        float *ws = static_cast<float *>(workspace);
        e = la::prefill_states(dt, Di, Mi, C, K, V, ws, (int)BH, (int)N, G, cps, G, s);
        if (e == hipSuccess) e = la::prefill_scan(ws, (int)BH, Di, Mi, G, G, S_out, z_out, s);
        if (e == hipSuccess)
            e = la::prefill_outputs(dt, Di, Mi, C, Q, K, V, out, ws, (int)BH, (int)N, G, cps, 0, nullptr, nullptr, s);
    }
    return hip_status(e);
}

LA_API size_t la_noalloc_scratch_bytes(void) { return kScratchBytes; }

LA_API int la_forward_chunked_noalloc(const void *Q, const void *K, const void *V, void *out, int64_t B,
                                      int64_t H, int64_t N, int64_t D, int64_t M, int causal, int dtype,
                                      int chunk_req, float *S_out, float *z_out, void *stream) {
    Plan p;
    int st = make_plan(B, H, N, D, M, causal, dtype, chunk_req, &p, 0, true);
    if (st != LA_OK) return st;
    if (p.ws_bytes > kScratchBytes) return LA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (p.ws_bytes > 0 && B * H > 0 && N > 0) {
        // the same argument checks as la_forward_chunked, before the scratch is touched
        if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_INVALID_ARG;
        if (S_out && (!aligned16(S_out) || !aligned16(z_out))) return LA_ERR_INVALID_ARG;
        if (!Q || !K || !V || !out) return LA_ERR_INVALID_ARG;
        if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(out)) return LA_ERR_INVALID_ARG;
        ws = device_scratch();
        if (ws == nullptr) return LA_ERR_HIP;
        if (causal) {
            // the look-back header and flags start at zero on every call (the kernels'
            // own workspace is at the front of the scratch for padded plans too); the
            // state slots are written before they are read
            const size_t words = la::kWsHeaderWords + la::fused_flag_words((long)(B * H) * p.segments);
            (void)hipGetLastError();
            if (la::fill_zero(static_cast<float *>(ws), words, as_stream(stream)) != hipSuccess) return LA_ERR_HIP;
        }
    }
    return la_forward_chunked(Q, K, V, out, B, H, N, D, M, causal, dtype, chunk_req, ws, ws ? kScratchBytes : 0,
                              S_out, z_out, stream);
}

LA_API int la_forward_continue(const void *Q, const void *K, const void *V, void *out, int64_t B, int64_t H,
                               int64_t N, int64_t D, int64_t M, int dtype, int chunk_req, const float *S_in,
                               const float *z_in, void *workspace, size_t workspace_bytes, float *S_out,
                               float *z_out, void *stream) {
    Plan p;
    int st = make_plan(B, H, N, D, M, 1, dtype, chunk_req, &p, 0, true);
    if (st != LA_OK) return st;
    if ((S_in == nullptr) != (z_in == nullptr)) return LA_ERR_INVALID_ARG;
    if (S_in && (!aligned16(S_in) || !aligned16(z_in))) return LA_ERR_INVALID_ARG;
    if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_INVALID_ARG;
    if (S_out && (!aligned16(S_out) || !aligned16(z_out))) return LA_ERR_INVALID_ARG;
    const int64_t BH = B * H;
    if (BH == 0) return LA_OK;
    hipStream_t s = as_stream(stream);
    if (N == 0) {
        if (S_out == nullptr) return LA_OK;
        (void)hipGetLastError();
        if (S_in == nullptr) {
            hipError_t e = la::fill_zero(S_out, (size_t)(BH * D * M), s);
            if (e == hipSuccess) e = la::fill_zero(z_out, (size_t)(BH * D), s);
            return hip_status(e);
        }
        hipError_t e = hipSuccess;
        if (S_out != S_in)
            e = hipMemcpyAsync(S_out, S_in, (size_t)(BH * D * M) * sizeof(float), hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess && z_out != z_in)
            e = hipMemcpyAsync(z_out, z_in, (size_t)(BH * D) * sizeof(float), hipMemcpyDeviceToDevice, s);
        return hip_status(e);
    }
    if (!Q || !K || !V || !out) return LA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(out)) return LA_ERR_INVALID_ARG;
    if (p.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < p.ws_bytes)) return LA_ERR_WORKSPACE;
    if (p.ws_bytes > 0 && !aligned16(workspace)) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    if (p.padded)
        return hip_status(run_padded(p, Q, K, V, out, BH, N, D, M, 1, dtype, workspace, S_in, z_in, S_out, z_out, s));
    const int dt = dtype, Di = (int)D, Mi = (int)M, C = p.chunk, G = p.segments, cps = p.chunks_per_segment;
    hipError_t e = p.onepass ? la::prefill_onepass(dt, Di, Mi, C, Q, K, V, out, workspace, (int)BH, (int)N, G, cps,
                                                   S_out, z_out, S_in, z_in, s)
                             : la::prefill_fused(dt, Di, Mi, C, Q, K, V, out, workspace, (int)BH, (int)N, G, cps,
                                                 S_out, z_out, S_in, z_in, s);
    return hip_status(e);
}

LA_API int la_workspace_status(const void *workspace, size_t workspace_bytes, void *stream) {
    if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < 16) return LA_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    unsigned word = 0;
    hipError_t e = hipMemcpyAsync(&word, static_cast<const unsigned *>(workspace) + la::kWsErrorWord, sizeof(word),
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return LA_ERR_HIP;
    return word == 0u ? LA_OK : LA_ERR_GAVE_UP;
}

LA_API int la_workspace_init(void *workspace, size_t workspace_bytes, void *stream) {
    if (workspace_bytes == 0) return LA_OK;
    if (workspace == nullptr || !aligned16(workspace) || workspace_bytes % 4 != 0) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(la::fill_zero(static_cast<float *>(workspace), workspace_bytes / 4, as_stream(stream)));
}

// ---- stage entry points ----------------------------------------------------

namespace {
int check_stage(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype, int chunk, int segments,
                size_t ws_bytes, const void *ws) {
    int st = check_shape(B, H, N, D, M, dtype);
    if (st != LA_OK) return st;
    if (chunk != 16 && chunk != 32 && chunk != 64) return LA_ERR_UNSUPPORTED;
    if (!la::prefill_supported(dtype, (int)D, (int)M, chunk)) return LA_ERR_UNSUPPORTED;
    if (segments < 1) return LA_ERR_INVALID_ARG;
    const int64_t n_chunks = (N + chunk - 1) / chunk;
    if (N > 0) {
        const int64_t cps = (n_chunks + segments - 1) / segments;
        // every segment must own at least one chunk
        if ((int64_t)(segments - 1) * cps >= n_chunks) return LA_ERR_UNSUPPORTED;
    }
    if ((int64_t)B * H * segments > INT_MAX / 256) return LA_ERR_UNSUPPORTED;
    const size_t need = state_ws_bytes(B * H, D, M, segments);
    if (ws == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    if (!aligned16(ws)) return LA_ERR_INVALID_ARG;
    return LA_OK;
}
int cps_of(int64_t N, int chunk, int segments) {
    const int64_t n_chunks = (N + chunk - 1) / chunk;
    return (int)((n_chunks + segments - 1) / segments);
}
}  // namespace

namespace {
// Shared validation and launch of the two explicit-plan causal entry points.
int forward_explicit(bool onepass, const void *Q, const void *K, const void *V, void *out, int64_t B, int64_t H,
                     int64_t N, int64_t D, int64_t M, int dtype, int chunk, int segments, const float *S_in,
                     const float *z_in, void *workspace, size_t workspace_bytes, float *S_out, float *z_out,
                     void *stream) {
    int st = check_shape(B, H, N, D, M, dtype);
    if (st != LA_OK) return st;
    if (chunk != 16 && chunk != 32 && chunk != 64) return LA_ERR_UNSUPPORTED;
    if (!la::prefill_supported(dtype, (int)D, (int)M, chunk)) return LA_ERR_UNSUPPORTED;
    if (onepass && !la::prefill_onepass_supported(dtype, (int)D, (int)M, chunk)) return LA_ERR_UNSUPPORTED;
    if (segments < 1) return LA_ERR_INVALID_ARG;
    if ((S_in == nullptr) != (z_in == nullptr)) return LA_ERR_INVALID_ARG;
    if (S_in && (!aligned16(S_in) || !aligned16(z_in))) return LA_ERR_INVALID_ARG;
    if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_INVALID_ARG;
    if (S_out && (!aligned16(S_out) || !aligned16(z_out))) return LA_ERR_INVALID_ARG;
    const int64_t BH = B * H;
    if (N > 0) {
        const int64_t n_chunks = (N + chunk - 1) / chunk;
        const int64_t cps = (n_chunks + segments - 1) / segments;
        if ((int64_t)(segments - 1) * cps >= n_chunks) return LA_ERR_UNSUPPORTED;
        if (onepass && cps > la::kOnePassMaxChunks) return LA_ERR_UNSUPPORTED;
    }
    if (BH * segments > INT_MAX / 256) return LA_ERR_UNSUPPORTED;
    const size_t need = segments > 1 ? la::fused_ws_bytes(BH, segments, (int)(D * M + D)) : 0;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return LA_ERR_INVALID_ARG;
    if (BH == 0) return LA_OK;
    hipStream_t s = as_stream(stream);
    if (N == 0) {
        if (S_out == nullptr) return LA_OK;
        (void)hipGetLastError();
        hipError_t e = hipSuccess;
        if (S_in == nullptr) {
            e = la::fill_zero(S_out, (size_t)(BH * D * M), s);
            if (e == hipSuccess) e = la::fill_zero(z_out, (size_t)(BH * D), s);
        } else {
            if (S_out != S_in)
                e = hipMemcpyAsync(S_out, S_in, (size_t)(BH * D * M) * sizeof(float), hipMemcpyDeviceToDevice, s);
            if (e == hipSuccess && z_out != z_in)
                e = hipMemcpyAsync(z_out, z_in, (size_t)(BH * D) * sizeof(float), hipMemcpyDeviceToDevice, s);
        }
        return hip_status(e);
    }
    if (!Q || !K || !V || !out) return LA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(out)) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    const int cps = cps_of(N, chunk, segments);
    return hip_status(onepass ? la::prefill_onepass(dtype, (int)D, (int)M, chunk, Q, K, V, out, workspace, (int)BH,
                                                    (int)N, segments, cps, S_out, z_out, S_in, z_in, s)
                              : la::prefill_fused(dtype, (int)D, (int)M, chunk, Q, K, V, out, workspace, (int)BH,
                                                  (int)N, segments, cps, S_out, z_out, S_in, z_in, s));
}
}  // namespace

LA_API int la_forward_fused(const void *Q, const void *K, const void *V, void *out, int64_t B, int64_t H,
                            int64_t N, int64_t D, int64_t M, int dtype, int chunk, int segments, const float *S_in,
                            const float *z_in, void *workspace, size_t workspace_bytes, float *S_out, float *z_out,
                            void *stream) {
    return forward_explicit(false, Q, K, V, out, B, H, N, D, M, dtype, chunk, segments, S_in, z_in, workspace,
                            workspace_bytes, S_out, z_out, stream);
}

LA_API int la_forward_onepass(const void *Q, const void *K, const void *V, void *out, int64_t B, int64_t H,
                              int64_t N, int64_t D, int64_t M, int dtype, int chunk, int segments, const float *S_in,
                              const float *z_in, void *workspace, size_t workspace_bytes, float *S_out, float *z_out,
                              void *stream) {
    return forward_explicit(true, Q, K, V, out, B, H, N, D, M, dtype, chunk, segments, S_in, z_in, workspace,
                            workspace_bytes, S_out, z_out, stream);
}

LA_API int la_segment_states(const void *K, const void *V, float *ws, size_t ws_bytes, int64_t B, int64_t H,
                             int64_t N, int64_t D, int64_t M, int dtype, int chunk, int segments, int nstates,
                             void *stream) {
    int st = check_stage(B, H, N, D, M, dtype, chunk, segments, ws_bytes, ws);
    if (st != LA_OK) return st;
    if (nstates != segments && nstates != segments - 1) return LA_ERR_INVALID_ARG;
    if (B * H == 0 || N == 0 || nstates == 0) return LA_OK;
    if (!K || !V || !aligned16(K) || !aligned16(V)) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(la::prefill_states(dtype, (int)D, (int)M, chunk, K, V, ws, (int)(B * H), (int)N, segments,
                                         cps_of(N, chunk, segments), nstates, as_stream(stream)));
}

LA_API int la_segment_scan(float *ws, size_t ws_bytes, int64_t B, int64_t H, int64_t D, int64_t M, int segments,
                           int nstates, float *S_out, float *z_out, void *stream) {
    if (B < 0 || H < 0) return LA_ERR_INVALID_ARG;
    if (!dim_ok(D) || !dim_ok(M)) return LA_ERR_UNSUPPORTED;
    if (segments < 1) return LA_ERR_INVALID_ARG;
    if (nstates != segments && nstates != segments - 1) return LA_ERR_INVALID_ARG;
    if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_INVALID_ARG;
    if (S_out && (!aligned16(S_out) || !aligned16(z_out))) return LA_ERR_INVALID_ARG;
    if (bh_over(B, H, INT_MAX / 8)) return LA_ERR_UNSUPPORTED;
    const size_t need = state_ws_bytes(B * H, D, M, segments);
    if (ws == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    if (!aligned16(ws)) return LA_ERR_INVALID_ARG;
    if (B * H == 0) return LA_OK;
    (void)hipGetLastError();
    return hip_status(la::prefill_scan(ws, (int)(B * H), (int)D, (int)M, segments, nstates, S_out, z_out,
                                       as_stream(stream)));
}

LA_API int la_segment_outputs(const void *Q, const void *K, const void *V, void *out, const float *ws,
                              size_t ws_bytes, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal,
                              int dtype, int chunk, int segments, float *S_out, float *z_out, void *stream) {
    int st = check_stage(B, H, N, D, M, dtype, chunk, segments, ws_bytes, ws);
    if (st != LA_OK) return st;
    if (causal != 0 && causal != 1) return LA_ERR_INVALID_ARG;
    if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_INVALID_ARG;
    if (S_out && (!aligned16(S_out) || !aligned16(z_out))) return LA_ERR_INVALID_ARG;
    if (B * H == 0 || N == 0) return LA_OK;
    if (!Q || !out || !aligned16(Q) || !aligned16(out)) return LA_ERR_INVALID_ARG;
    if (causal && (!K || !V || !aligned16(K) || !aligned16(V))) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(la::prefill_outputs(dtype, (int)D, (int)M, chunk, Q, K, V, out, ws, (int)(B * H), (int)N,
                                          segments, cps_of(N, chunk, segments), causal, causal ? S_out : nullptr,
                                          causal ? z_out : nullptr, as_stream(stream)));
}

// ---- recurrent mode ---------------------------------------------------------

LA_API int la_decode_step(float *S, float *z, const void *q, const void *k, const void *v, float *out, int64_t B,
                          int64_t H, int64_t D, int64_t M, int dtype, void *stream) {
    if (B < 0 || H < 0) return LA_ERR_INVALID_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16 && dtype != LA_F32_FEATURES) return LA_ERR_INVALID_ARG;
    if (!dim_padded_ok(D) || !dim_padded_ok(M)) return LA_ERR_UNSUPPORTED;
    if (bh_over(B, H, INT_MAX)) return LA_ERR_UNSUPPORTED;
    if (B * H == 0) return LA_OK;
    if (!S || !z || !q || !k || !v || !out) return LA_ERR_INVALID_ARG;
    if (!aligned16(S) || !aligned16(z) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    if (!dim_ok(D) || !dim_ok(M))
        return hip_status(la::decode_any(dtype, (int)D, (int)M, S, z, q, k, v, out, (int)(B * H), 1,
                                         as_stream(stream)));
    return hip_status(la::decode_step(dtype, (int)D, (int)M, S, z, q, k, v, out, (int)(B * H), as_stream(stream)));
}

LA_API int la_decode_step_features(float *S, float *z, const void *q, const void *k, const void *v, float *out,
                                   int64_t B, int64_t H, int64_t D, int64_t M, int dtype, const float *W, int64_t F,
                                   int kind, int flags, void *stream) {
    if (B < 0 || H < 0) return LA_ERR_INVALID_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
    if (kind != LA_FEATURE_PRF && kind != LA_FEATURE_TRF) return LA_ERR_INVALID_ARG;
    if ((flags & ~LA_FEATURE_NORMALIZE) != 0) return LA_ERR_INVALID_ARG;
    if (!dim_ok(D) || !dim_ok(M) || !(F == 16 || F == 32 || F == 64)) return LA_ERR_UNSUPPORTED;
    if (bh_over(B, H, INT_MAX)) return LA_ERR_UNSUPPORTED;
    if (B * H == 0) return LA_OK;
    if (!S || !z || !q || !k || !v || !out || !W) return LA_ERR_INVALID_ARG;
    if (!aligned16(S) || !aligned16(z) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        !aligned16(W))
        return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(la::decode_step_features(dtype, (int)D, (int)F, (int)M, S, z, q, k, v, out, W, kind,
                                               (flags & LA_FEATURE_NORMALIZE) != 0, (int)(B * H),
                                               as_stream(stream)));
}

namespace {
// Backward plan: chunks of kBackwardChunk positions, segments sized like the
// forward planner's (about 512 workgroups, or 256 for states above 64 x 64).
struct BwdPlan {
    int G = 0, cps = 0;
    size_t states_bytes = 0, den_bytes = 0, ws_bytes = 0;
};
int bwd_plan(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype, BwdPlan *p) {
    // the gradient is taken through phi = elu + 1, or (LA_F32_FEATURES) with respect
    // to the features themselves; gradients are fp32
    if (dtype & LA_OUT_BF16) return LA_ERR_UNSUPPORTED;
    int st = check_shape(B, H, N, D, M, dtype);
    if (st != LA_OK) return st;
    const int64_t BH = B * H;
    if (BH == 0 || N == 0) return LA_OK;
    const int C = la::kBackwardChunk;
    if (!la::prefill_supported(dtype, (int)D, (int)M, C)) return LA_ERR_UNSUPPORTED;
    const int64_t n_chunks = (N + C - 1) / C;
    const int64_t target_wg = (D * M <= 4096) ? 512 : 256;
    int64_t cps = (n_chunks * BH + target_wg - 1) / target_wg;
    if (cps < 1) cps = 1;
    int64_t G = (n_chunks + cps - 1) / cps;
    cps = (n_chunks + G - 1) / G;
    G = (n_chunks + cps - 1) / cps;
    if (BH * G > INT_MAX / 256) return LA_ERR_UNSUPPORTED;
    p->G = (int)G;
    p->cps = (int)cps;
    p->states_bytes = state_ws_bytes(BH, D, M, (int)G);
    p->den_bytes = ((size_t)(BH * N) * sizeof(float) + 255) / 256 * 256;
    p->ws_bytes = 2 * p->states_bytes + p->den_bytes;
    return LA_OK;
}
}  // namespace

LA_API size_t la_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype) {
    BwdPlan p;
    return bwd_plan(B, H, N, D, M, dtype, &p) == LA_OK ? p.ws_bytes : 0;
}

LA_API int la_backward_chunked(const void *Q, const void *K, const void *V, const float *out, const float *dout,
                               float *dQ, float *dK, float *dV, int64_t B, int64_t H, int64_t N, int64_t D,
                               int64_t M, int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    BwdPlan p;
    int st = bwd_plan(B, H, N, D, M, dtype, &p);
    if (st != LA_OK) return st;
    const int64_t BH = B * H;
    if (BH == 0 || N == 0) return LA_OK;
    if (!Q || !K || !V || !out || !dout || !dQ || !dK || !dV) return LA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(out) || !aligned16(dout) || !aligned16(dQ) ||
        !aligned16(dK) || !aligned16(dV))
        return LA_ERR_INVALID_ARG;
    if (workspace == nullptr || workspace_bytes < p.ws_bytes) return LA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LA_ERR_INVALID_ARG;
    unsigned char *w = static_cast<unsigned char *>(workspace);
    float *fwd_ws = reinterpret_cast<float *>(w);
    float *rev_ws = reinterpret_cast<float *>(w + p.states_bytes);
    float *den = reinterpret_cast<float *>(w + 2 * p.states_bytes);
    const int C = la::kBackwardChunk, G = p.G, cps = p.cps, Di = (int)D, Mi = (int)M, E = (int)(D * M + D);
    hipStream_t s = as_stream(stream);
    (void)hipGetLastError();
    hipError_t e = hipSuccess;
    if (G > 1) {
        e = la::prefill_states(dtype, Di, Mi, C, K, V, fwd_ws, (int)BH, (int)N, G, cps, G - 1, s);
        if (e == hipSuccess) e = la::prefill_scan(fwd_ws, (int)BH, Di, Mi, G, G - 1, nullptr, nullptr, s);
    }
    if (e == hipSuccess)
        e = la::backward_dq(dtype, Di, Mi, Q, K, V, out, dout, fwd_ws, rev_ws, den, dQ, (int)BH, (int)N, G, cps, s);
    if (e == hipSuccess && G > 1) e = la::backward_rev_scan(rev_ws, (int)BH, E, G, s);
    if (e == hipSuccess)
        e = la::backward_dkv(dtype, Di, Mi, Q, K, V, out, dout, rev_ws, den, dK, dV, (int)BH, (int)N, G, cps, s);
    return hip_status(e);
}

namespace {
int scan_check(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype, int64_t *items) {
    if (B < 0 || H < 0 || N < 0) return LA_ERR_INVALID_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
    if (!dim_ok(D) || !dim_ok(M)) return LA_ERR_UNSUPPORTED;
    if (N > INT_MAX || bh_over(B, H, INT_MAX / 8)) return LA_ERR_UNSUPPORTED;
    const int64_t R = la::softmax_scan_rows((int)M);
    const int64_t NS = (N + R - 1) / R;
    if (B * H * NS > INT_MAX / 64) return LA_ERR_UNSUPPORTED;
    *items = B * H * NS;
    return LA_OK;
}
}  // namespace

LA_API size_t la_softmax_scan_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M) {
    int64_t items = 0;
    if (scan_check(B, H, N, D, M, LA_F32, &items) != LA_OK) return 0;
    const int64_t NS = B * H > 0 ? items / (B * H) : 0;
    return NS > 1 ? la::scan_ws_bytes((long)items, (int)M) : 0;
}

LA_API int la_softmax_scan(const void *q, const void *K, const void *V, float *out, int64_t B, int64_t H,
                           int64_t N, int64_t D, int64_t M, int dtype, void *workspace, size_t workspace_bytes,
                           float *m_out, float *u_out, float *w_out, void *stream) {
    int64_t items = 0;
    int st = scan_check(B, H, N, D, M, dtype, &items);
    if (st != LA_OK) return st;
    if ((m_out == nullptr) != (u_out == nullptr) || (m_out == nullptr) != (w_out == nullptr)) return LA_ERR_INVALID_ARG;
    if (w_out && !aligned16(w_out)) return LA_ERR_INVALID_ARG;
    if (B * H == 0 || N == 0) return LA_OK;
    if (!q || !K || !V || !out) return LA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(out)) return LA_ERR_INVALID_ARG;
    const size_t need = la_softmax_scan_workspace_bytes(B, H, N, D, M);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(la::softmax_scan(dtype, (int)D, (int)M, q, K, V, out, workspace, (int)(B * H), (int)N, m_out,
                                       u_out, w_out, as_stream(stream)));
}

LA_API int la_softmax_step(float *m, float *u, float *w, const void *q, const void *k, const void *v, float *out,
                           int64_t B, int64_t H, int64_t D, int64_t M, int dtype, void *stream) {
    if (B < 0 || H < 0) return LA_ERR_INVALID_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
    if (!dim_ok(D) || !dim_ok(M)) return LA_ERR_UNSUPPORTED;
    if (bh_over(B, H, INT_MAX)) return LA_ERR_UNSUPPORTED;
    if (B * H == 0) return LA_OK;
    if (!m || !u || !w || !q || !k || !v || !out) return LA_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(la::softmax_step(dtype, (int)D, (int)M, m, u, w, q, k, v, out, (int)(B * H),
                                       as_stream(stream)));
}

LA_API int la_decode_steps(float *S, float *z, const void *q, const void *k, const void *v, float *out, int64_t B,
                           int64_t H, int64_t T, int64_t D, int64_t M, int dtype, void *stream) {
    if (B < 0 || H < 0 || T < 0) return LA_ERR_INVALID_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16 && dtype != LA_F32_FEATURES) return LA_ERR_INVALID_ARG;
    if (!dim_padded_ok(D) || !dim_padded_ok(M)) return LA_ERR_UNSUPPORTED;
    if (bh_over(B, H, INT_MAX) || T > INT_MAX) return LA_ERR_UNSUPPORTED;
    if (B * H > 0 && T > INT64_MAX / (B * H * (D > M ? D : M))) return LA_ERR_UNSUPPORTED;
    if (B * H == 0 || T == 0) return LA_OK;
    if (!S || !z || !q || !k || !v || !out) return LA_ERR_INVALID_ARG;
    if (!aligned16(S) || !aligned16(z) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    hipStream_t s = as_stream(stream);
    if (!dim_ok(D) || !dim_ok(M))
        return hip_status(la::decode_any(dtype, (int)D, (int)M, S, z, q, k, v, out, (int)(B * H), (int)T, s));
    // From about a dozen tokens on, the chunked causal kernels (MFMA tiles, the state
    // carried in and out in place) beat the register recurrence.  They are used when
    // every head is one segment, i.e. when no workspace is needed.
    // (fp32 inputs only: with bf16 inputs the chunked kernels round MFMA operands to
    // bf16, while this entry point keeps fp32 arithmetic for both input types)
    if (dtype != LA_BF16 && decode_steps_chunked(T, D, M)) {
        Plan p;
        if (make_plan(B, H, T, D, M, 1, dtype, 16, &p) == LA_OK && p.ws_bytes == 0 && p.segments == 1) {
            const int BH = (int)(B * H), Di = (int)D, Mi = (int)M;
            hipError_t e = p.onepass ? la::prefill_onepass(dtype, Di, Mi, 16, q, k, v, out, nullptr, BH, (int)T, 1,
                                                           p.chunks_per_segment, S, z, S, z, s)
                                     : la::prefill_fused(dtype, Di, Mi, 16, q, k, v, out, nullptr, BH, (int)T, 1,
                                                         p.chunks_per_segment, S, z, S, z, s);
            return hip_status(e);
        }
    }
    return hip_status(la::decode_steps(dtype, (int)D, (int)M, S, z, q, k, v, out, (int)(B * H), (int)T, s));
}

// ---- causal attention with the random-feature map fused ----------------------

namespace {
// The plan of la_forward_features (LA_OK only when the fused kernel runs it).
int features_plan(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int64_t F, int causal, Plan *p) {
    if (causal != 0 && causal != 1) return LA_ERR_INVALID_ARG;
    if (!dim_ok(D) || !dim_ok(F)) return LA_ERR_UNSUPPORTED;
    // the fused kernels' LDS (raw rows and W besides the attention tiles) admits
    // two workgroups per CU: plan 512 resident workgroups
    int st = make_plan(B, H, N, F, M, causal, LA_F32_FEATURES, la::kFusedFeatureChunk, p, 512);
    if (st != LA_OK) return st;
    if (B * H == 0 || N == 0) return LA_OK;
    if (!causal) return la::prefill_features_noncausal_supported((int)D, (int)F, (int)M) ? LA_OK : LA_ERR_UNSUPPORTED;
    // the one-pass kernel where its segments fit (at most four chunks) and its LDS
    // does; otherwise two launches: the map into the workspace, then the attention
    // kernels on the features.  (The fused two-phase kernel forms the projections of
    // the k rows in both of its phases, and measured slower than the two launches:
    // 204 against 193 us at B1 H8 N65536 D64 F16 M64, 56.9 against 51.5 us at
    // B8 H8 N1024 D64 F64 M64.)
    if (p->onepass && !la::prefill_features_onepass_supported((int)D, (int)F, (int)M)) p->onepass = false;
    if (!p->onepass) {
        Plan a;
        st = make_plan(B, H, N, F, M, 1, LA_F32_FEATURES, 0, &a);
        if (st != LA_OK) return st;
        const size_t rows = (size_t)(B * H) * (size_t)N;
        p->split = true;
        p->att_chunk = a.chunk;
        p->att_segments = a.segments;
        p->att_cps = a.chunks_per_segment;
        p->att_onepass = a.onepass;
        // the attention's look-back header stays at the front of the workspace
        size_t off = round256(a.ws_bytes > 256 ? a.ws_bytes : 256);
        p->inner_ws = a.ws_bytes;
        p->oQ = off;
        off += round256(rows * (size_t)F * 4);
        p->oK = off;
        off += round256(rows * (size_t)F * 4);
        p->oV = off;  // bf16 V widened (fp32 V is read in place)
        off += round256(rows * (size_t)M * 4);
        p->ws_bytes = off;
    }
    return LA_OK;
}
}  // namespace

LA_API size_t la_forward_features_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int64_t F,
                                                  int causal) {
    Plan p;
    // a supported shape asks for at least 256 bytes, so 0 always means "refused"
    return features_plan(B, H, N, D, M, F, causal, &p) == LA_OK ? std::max<size_t>(p.ws_bytes, 256) : 0;
}

LA_API int la_forward_features(const void *Q, const void *K, const void *V, float *out, int64_t B, int64_t H,
                               int64_t N, int64_t D, int64_t M, int causal, int dtype, const float *W, int64_t F,
                               int kind, int flags, void *workspace, size_t workspace_bytes, const float *S_in,
                               const float *z_in, float *S_out, float *z_out, void *stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
    if (kind != LA_FEATURE_PRF && kind != LA_FEATURE_TRF) return LA_ERR_INVALID_ARG;
    if ((flags & ~LA_FEATURE_NORMALIZE) != 0) return LA_ERR_INVALID_ARG;
    if (causal == 0 && (S_in || z_in || S_out || z_out)) return LA_ERR_INVALID_ARG;  // states: causal only
    Plan p;
    int st = features_plan(B, H, N, D, M, F, causal, &p);
    if (st != LA_OK) return st;
    if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_INVALID_ARG;
    if ((S_in == nullptr) != (z_in == nullptr)) return LA_ERR_INVALID_ARG;
    if (S_out && (!aligned16(S_out) || !aligned16(z_out))) return LA_ERR_INVALID_ARG;
    if (S_in && (!aligned16(S_in) || !aligned16(z_in))) return LA_ERR_INVALID_ARG;
    const int64_t BH = B * H;
    if (BH == 0) return LA_OK;
    hipStream_t s = as_stream(stream);
    if (N == 0) {
        if (S_out == nullptr) return LA_OK;
        (void)hipGetLastError();
        hipError_t e = hipSuccess;
        if (S_in) {  // the state passes through unchanged
            if (S_out != S_in)
                e = hipMemcpyAsync(S_out, S_in, (size_t)(BH * F * M) * sizeof(float), hipMemcpyDeviceToDevice, s);
            if (e == hipSuccess && z_out != z_in)
                e = hipMemcpyAsync(z_out, z_in, (size_t)(BH * F) * sizeof(float), hipMemcpyDeviceToDevice, s);
        } else {
            e = la::fill_zero(S_out, (size_t)(BH * F * M), s);
            if (e == hipSuccess) e = la::fill_zero(z_out, (size_t)(BH * F), s);
        }
        return hip_status(e);
    }
    if (!Q || !K || !V || !out || !W) return LA_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(out) || !aligned16(W)) return LA_ERR_INVALID_ARG;
    if (p.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < p.ws_bytes)) return LA_ERR_WORKSPACE;
    if (p.ws_bytes > 0 && !aligned16(workspace)) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    const int norm = (flags & LA_FEATURE_NORMALIZE) != 0;
    if (p.split) {
        unsigned char *w = static_cast<unsigned char *>(workspace);
        float *fq = reinterpret_cast<float *>(w + p.oQ), *fk = reinterpret_cast<float *>(w + p.oK);
        const int dt = dtype == LA_F32 ? la::kDtypeF32 : la::kDtypeBf16;
        hipError_t e = la::feature_map(dt, (int)D, (int)F, kind, Q, fq, K, fk, W, (long)(BH * N), norm != 0, s);
        const void *Vf = V;
        if (e == hipSuccess && dtype == LA_BF16) {
            float *vw = reinterpret_cast<float *>(w + p.oV);
            e = la::widen_bf16(V, vw, (long)(BH * N * M), s);
            Vf = vw;
        }
        void *iw = p.inner_ws > 0 ? workspace : nullptr;
        const int Fi = (int)F, Mi = (int)M, C = p.att_chunk, G = p.att_segments, cps = p.att_cps;
        if (e == hipSuccess)
            e = p.att_onepass ? la::prefill_onepass(LA_F32_FEATURES, Fi, Mi, C, fq, fk, Vf, out, iw, (int)BH, (int)N, G,
                                                    cps, S_out, z_out, S_in, z_in, s)
                              : la::prefill_fused(LA_F32_FEATURES, Fi, Mi, C, fq, fk, Vf, out, iw, (int)BH, (int)N, G,
                                                  cps, S_out, z_out, S_in, z_in, s);
        return hip_status(e);
    }
    if (!causal)
        return hip_status(la::prefill_features_noncausal(dtype == LA_F32 ? la::kDtypeF32 : la::kDtypeBf16, (int)D,
                                                         (int)F, (int)M, Q, K, V, W, kind, norm, out,
                                                         static_cast<float *>(workspace), (int)BH, (int)N, p.segments,
                                                         p.chunks_per_segment, s));
    return hip_status(dtype == LA_F32
                          ? la::prefill_features_f32((int)D, (int)F, (int)M, Q, K, V, W, kind, norm, out,
                                                     workspace, (int)BH, (int)N, p.segments, p.chunks_per_segment,
                                                     S_out, z_out, S_in, z_in, s)
                          : la::prefill_features_bf16((int)D, (int)F, (int)M, Q, K, V, W, kind, norm, out,
                                                      workspace, (int)BH, (int)N, p.segments, p.chunks_per_segment,
                                                      S_out, z_out, S_in, z_in, s));
}

// ---- feature maps ----------------------------------------------------------

LA_API int la_feature_map_backward(float *dX, const void *X, const float *dOut, int64_t rows, int64_t D, int dtype,
                                   const float *W, int64_t F, int kind, int flags, void *stream) {
    if (rows < 0 || D <= 0 || F <= 0) return LA_ERR_INVALID_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
    if (kind != LA_FEATURE_ELU && kind != LA_FEATURE_PRF && kind != LA_FEATURE_TRF) return LA_ERR_INVALID_ARG;
    if ((flags & ~LA_FEATURE_NORMALIZE) != 0) return LA_ERR_INVALID_ARG;
    if (kind == LA_FEATURE_ELU && F != D) return LA_ERR_INVALID_ARG;
    if (!dim_ok(D) || !dim_ok(F)) return LA_ERR_UNSUPPORTED;
    if (rows > INT64_MAX / 256) return LA_ERR_UNSUPPORTED;
    if (rows == 0) return LA_OK;
    if (!dX || !X || !dOut || (kind != LA_FEATURE_ELU && !W)) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(la::feature_map_backward(dtype, (int)D, (int)F, kind, X, dOut, W, dX, (long)rows,
                                               (flags & LA_FEATURE_NORMALIZE) != 0, as_stream(stream)));
}

LA_API int la_feature_map(float *out, const void *X, float *out2, const void *X2, int64_t rows, int64_t D,
                          int dtype, const float *W, int64_t F, int kind, int flags, void *stream) {
    if (rows < 0 || D <= 0 || F <= 0) return LA_ERR_INVALID_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
    if (kind != LA_FEATURE_ELU && kind != LA_FEATURE_PRF && kind != LA_FEATURE_TRF) return LA_ERR_INVALID_ARG;
    if ((flags & ~LA_FEATURE_NORMALIZE) != 0) return LA_ERR_INVALID_ARG;
    if (kind == LA_FEATURE_ELU && F != D) return LA_ERR_INVALID_ARG;
    if (!dim_ok(D) || !dim_ok(F)) return LA_ERR_UNSUPPORTED;
    if (rows > INT64_MAX / 256) return LA_ERR_UNSUPPORTED;
    if ((rows + 63) / 64 > INT_MAX) return LA_ERR_UNSUPPORTED;
    if ((X2 == nullptr) != (out2 == nullptr)) return LA_ERR_INVALID_ARG;
    if (rows == 0) return LA_OK;
    if (!out || !X || (kind != LA_FEATURE_ELU && !W)) return LA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(X) || (X2 && (!aligned16(X2) || !aligned16(out2)))) return LA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(la::feature_map(dtype, (int)D, (int)F, kind, X, out, X2, out2, W, (long)rows,
                                      (flags & LA_FEATURE_NORMALIZE) != 0, as_stream(stream)));
}

}  // extern "C"
