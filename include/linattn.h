/*
 * linattn -- causal kernelized linear attention on AMD Instinct MI355X (gfx950).
 *
 * Method: "Transformers are RNNs: Fast Autoregressive Transformers with Linear
 * Attention" (Katharopoulos et al., 2020), page of that title:
 *   - Proposed method: the softmax similarity is replaced by phi(q)^T phi(k);
 *     associativity gives phi(Q) (phi(K)^T V) with the sum computed once;
 *     causal masking is kept by the cumulative sums S_i, Z_i, updated step by
 *     step; the causal model is an RNN with the two memories (S, z).
 *   - Main findings: phi is elu based: phi(x) = elu(x) + 1, i.e. x + 1 for x > 0
 *     and exp(x) otherwise.
 *   With S_i = sum_{j<=i} phi(k_j) v_j^T (D x M) and z_i = sum_{j<=i} phi(k_j) (D):
 *     out_i = phi(q_i)^T S_i / (phi(q_i)^T z_i)        (causal)
 *     out_i = phi(q_i)^T S_{N-1} / (phi(q_i)^T z_{N-1}) (non-causal)
 *   No 1/sqrt(D) scaling and no epsilon in the denominator (phi > 0 keeps it positive).
 *
 * Conventions for every entry point:
 *   - Tensors are dense, row major, contiguous, in device memory owned by the
 *     caller; the library never allocates, frees or keeps a pointer.
 *     Q, K: [B][H][N][D]; V, out: [B][H][N][M]; S: [B][H][D][M]; z: [B][H][D].
 *   - Input element type: LA_F32 (float) or LA_BF16 (bfloat16 bit patterns,
 *     uint16).  Arithmetic and accumulation are fp32; out, S and z are fp32
 *     (out bf16 with LA_BF16 | LA_OUT_BF16, see la_dtype).
 *   - D and M must each be 16, 32, 64 or 128, except where an entry point
 *     says otherwise: la_forward_plan, la_forward_workspace_bytes,
 *     la_forward_chunked, la_forward_continue, la_decode_step and
 *     la_decode_steps take any multiple of 16 up to 128 (see "Widths without a
 *     kernel of their own" below).  All device pointers must be 16-byte
 *     aligned.  Outputs must not alias inputs.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting.  Concurrent calls that share a
 *     workspace race; calls with separate workspaces are thread safe.
 *   - Every call validates all arguments before it enqueues anything; on error
 *     it returns a status below and writes nothing.  It never aborts and never
 *     throws.  LA_ERR_HIP reports a launch failure from the HIP runtime.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define LA_API __attribute__((visibility("default")))
#else
#define LA_API
#endif

enum la_status {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = 1, /* null pointer, negative size, misalignment, bad flag */
    LA_ERR_UNSUPPORTED = 2, /* D, M, chunk or segment count outside the supported set */
    LA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    LA_ERR_HIP = 4,         /* the HIP runtime reported an error at launch */
    LA_ERR_GAVE_UP = 5      /* la_workspace_status: a look-back wait gave up (NaN rows written) */
};

/* LA_F32_FEATURES: fp32 Q and K rows that already hold the features phi(q),
 * phi(k) (for example from la_feature_map); the kernels then apply no feature
 * map, D is the feature dimension, and V is fp32.  Accepted by the forward
 * entry points, the segment stages, the decode entry points and
 * la_backward_chunked (which then returns the gradients with respect to the
 * features); not by the softmax scan. */
/* LA_BF16 | LA_OUT_BF16: bf16 inputs and bf16 outputs.  The forward entry
 * points (la_forward_chunked, la_forward_continue, la_forward_fused,
 * la_forward_onepass, la_segment_outputs; la_segment_states ignores the flag)
 * then write out as bf16 bit patterns, each the fp32 result rounded to nearest
 * even; arithmetic, S and z stay fp32.  Other entry points reject it. */
enum la_dtype { LA_F32 = 0, LA_BF16 = 1, LA_F32_FEATURES = 2, LA_OUT_BF16 = 16 };

/*
 * Widths without a kernel of their own (D or M of 48, 80, 96 or 112).  The
 * page's statement (page "Transformers are RNNs", Proposed method: the
 * similarity is the dot product phi(q)^T phi(k) of feature vectors of any
 * length) holds for every width; the kernels are built for 16, 32, 64 and 128.
 * la_forward_chunked and la_forward_continue run other multiples of 16 on
 * copies padded to the next of those widths, held in the workspace: Q and K
 * columns beyond D are -inf, which phi maps to exactly 0 (0 for
 * LA_F32_FEATURES inputs), V columns beyond M are 0, and only the first M
 * output columns and the [D][M] corner of the state are copied back.  The
 * workspace (la_forward_workspace_bytes) then also holds those copies, and such
 * calls move about twice the bytes of a call at a kernel width.  la_decode_step
 * and la_decode_steps run them on one generic kernel with the widths as
 * arguments (no workspace).  Results are those of the same problem at any
 * width: the extra features and values add exact zeros.
 */

/* Human-readable name of a status code (static string; never NULL). */
LA_API const char *la_status_str(int status);

/* Library version as major*10000 + minor*100 + patch. */
LA_API int la_version(void);

/*
 * Execution plan of the parallel (prefill) mode.
 *
 * The sequence of each (b, h) is cut into chunks of `chunk` positions, and the
 * chunks into `segments` contiguous groups of whole chunks.  Inside a chunk the
 * masked quadratic term phi(Q_c) phi(K_c)^T V_c is formed directly; across
 * chunks the running state (S, z) carries the sums (page "Transformers are
 * RNNs", Proposed method: cumulative sums updated step by step, sum computed
 * once and reused).  Segments are walked in parallel; an exclusive prefix over
 * their summed states links them.
 *
 * chunk_req: 0 = automatic, else 16, 32 or 64.  On LA_OK writes the chosen chunk,
 * the segment count and the workspace size (bytes) that la_forward_chunked
 * needs.  Pure host computation; makes no HIP call.  Any output pointer may be NULL.
 */
LA_API int la_forward_plan(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                           int causal, int dtype, int chunk_req,
                           int *chunk_out, int *segments_out, size_t *workspace_bytes_out);

/* Workspace bytes la_forward_chunked needs for these arguments (0 on invalid
 * arguments).  `causal` is an argument because the two modes keep different
 * workspaces: causal calls keep look-back flags and two states per segment,
 * non-causal calls one state per segment plus the total. */
LA_API size_t la_forward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                         int causal, int dtype, int chunk_req);

/*
 * Parallel-mode attention (prefill / training forward).
 *
 * causal = 1: out_i uses positions j <= i (diagonal included); one kernel
 *   whose workgroups (one per segment) pass summed states forward with a
 *   decoupled look-back: the one-pass kernel (la_forward_onepass) when the
 *   plan's segments hold at most 4 chunks, else the two-phase fused kernel
 *   (la_forward_fused).
 * causal = 0: every out_i uses all N positions (three stage kernels).
 * out: [B][H][N][M] fp32, fully written.
 * workspace: device memory of at least la_forward_workspace_bytes(...) bytes
 *   (NULL allowed when that size is 0).  Causal calls keep counters and flags
 *   in it: it must be zeroed (la_workspace_init) before its first use and
 *   again before it is used with a different plan (B*H, N, D, M, dtype or
 *   chunk); every completed call leaves it ready for the next call with the
 *   same plan.  Calls that run concurrently must not share a workspace.
 *   A segment waits for earlier segments of its head with a bounded wait (about
 *   4 million polls).  Workgroups are dispatched in segment order, so the wait
 *   ends unless the GPU is shared so heavily that earlier segments cannot run;
 *   if it gives up, the affected outputs (and S_out, z_out) are NaN, a nonzero
 *   error word is left in the workspace (32-bit word 3, byte offset 12), and
 *   the workspace must be zeroed again before its next use.  Word 4 (byte
 *   offset 16), when nonzero, caps each wait at that many polls; it exists so
 *   that tests can force the give-up path, and la_workspace_init clears it.
 * S_out [B][H][D][M], z_out [B][H][D]: optional (NULL to skip; both or neither);
 *   receive the final state S_{N-1}, z_{N-1}, so that la_decode_step can
 *   continue the sequence.
 * N = 0 or B*H = 0 is a valid empty call (with N = 0 and S_out given, the state
 * is written as zeros).
 */
LA_API int la_forward_chunked(const void *Q, const void *K, const void *V, void *out,
                              int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                              int causal, int dtype, int chunk_req,
                              void *workspace, size_t workspace_bytes,
                              float *S_out, float *z_out, void *stream);

/*
 * la_forward_chunked without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The call allocates nothing: the
 * workspace is a file-scope device array of la_noalloc_scratch_bytes() bytes
 * (LA_NOALLOC_SCRATCH_BYTES, 64 MiB) that every device using the library holds
 * until the process ends.  Arguments, results and errors as for
 * la_forward_chunked, plus LA_ERR_WORKSPACE when the plan needs more workspace
 * than the scratch holds (for example B*H = 16, N = 65536, D = M = 128 bf16
 * needs about 34 MB; a width padded to a kernel width also needs room for the
 * padded copies).  A causal call first clears the look-back header and flags
 * of the scratch with a fill kernel on `stream`, then runs la_forward_chunked's
 * kernels on it.  All calls on one device share that device's scratch: calls
 * that overlap in time on one device (another stream, another thread) race
 * and must be serialised by the caller.
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
LA_API size_t la_noalloc_scratch_bytes(void);
LA_API int la_forward_chunked_noalloc(const void *Q, const void *K, const void *V, void *out,
                                      int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                      int causal, int dtype, int chunk_req,
                                      float *S_out, float *z_out, void *stream);

/*
 * Causal attention continuing a sequence from a carried state: the positions
 * of this call come after earlier ones whose state is (S_in, z_in), so
 *   out_i = phi(q_i)^T (S_in + S_i) / phi(q_i)^T (z_in + z_i)
 * with S_i, z_i summed over this call's positions j <= i (page "Transformers
 * are RNNs", Proposed method: the causal model is an RNN whose memories S and z
 * carry every earlier position, so a sequence can be processed in pieces).
 * S_in [B][H][D][M], z_in [B][H][D] fp32: both, or neither (then the state is
 * zero and the call equals la_forward_chunked with causal = 1).  S_out / z_out
 * receive the state after the last position; they may be S_in / z_in
 * themselves (in-place continuation).  Plan, chunk_req and workspace as for
 * la_forward_chunked with causal = 1 (la_forward_workspace_bytes(..., 1, ...)).
 * With N = 0, S_out / z_out receive a copy of S_in / z_in (zeros without them).
 */
LA_API int la_forward_continue(const void *Q, const void *K, const void *V, void *out,
                               int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                               int dtype, int chunk_req,
                               const float *S_in, const float *z_in,
                               void *workspace, size_t workspace_bytes,
                               float *S_out, float *z_out, void *stream);

/* Zero a workspace (an enqueued fill kernel; graph-capture safe). bytes % 4 == 0. */
LA_API int la_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/*
 * Whether a look-back wait gave up in the calls that used this workspace since
 * it was last zeroed (causal la_forward_chunked, la_forward_continue,
 * la_forward_fused, la_forward_onepass, la_softmax_scan): waits for `stream`
 * (every call enqueued on it so far completes), then reads the error word
 * (32-bit word 3).  Returns LA_OK when no wait gave up, LA_ERR_GAVE_UP when one
 * did (the affected outputs and final states are NaN; zero the workspace with
 * la_workspace_init before its next use), LA_ERR_INVALID_ARG for a NULL or
 * misaligned workspace or fewer than 16 bytes, LA_ERR_HIP if the copy or the
 * wait fails.  Blocks the calling thread; not for use under graph capture.
 */
LA_API int la_workspace_status(const void *workspace, size_t workspace_bytes, void *stream);

/*
 * The causal fused kernel of la_forward_chunked with an explicit plan: chunk
 * (16, 32 or 64) and segments (each segment must own at least one chunk).
 * Workspace: 0 bytes when segments == 1, else
 *   (64 + 64*ceil(B*H*segments/64)) * 4 + 2 * B*H*segments * P * 4 bytes with
 *   P = 64*ceil((D*M + D)/64) (one state padded to whole 256-byte blocks),
 * initialised as for la_forward_chunked.  S_in / z_in as for la_forward_continue
 * (NULL: start from zero); S_out / z_out as for la_forward_chunked.
 */
LA_API int la_forward_fused(const void *Q, const void *K, const void *V, void *out,
                            int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                            int dtype, int chunk, int segments,
                            const float *S_in, const float *z_in,
                            void *workspace, size_t workspace_bytes,
                            float *S_out, float *z_out, void *stream);

/*
 * The causal one-pass kernel of la_forward_chunked with an explicit plan:
 * chunk (16, 32 or 64) and segments, each segment owning at least one and at
 * most 4 chunks (LA_ERR_UNSUPPORTED otherwise, or when the kernel's LDS does
 * not fit this (D, M, chunk)).  Each workgroup reads its segment's Q, K, V
 * once, keeps its unnormalised rows on chip while it publishes its segment
 * state and looks back for the prefix of the earlier segments, then writes
 * out = (num + phi(q) S_prefix) / (den + phi(q) . z_prefix)  (page
 * "Transformers are RNNs", Proposed method: the same cumulative sums, split
 * at the segment start).  Workspace size and initialisation as for
 * la_forward_fused (the two kernels share the format, not a live workspace).
 * S_in / z_in as for la_forward_continue (NULL: start from zero).
 */
LA_API int la_forward_onepass(const void *Q, const void *K, const void *V, void *out,
                              int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                              int dtype, int chunk, int segments,
                              const float *S_in, const float *z_in,
                              void *workspace, size_t workspace_bytes,
                              float *S_out, float *z_out, void *stream);

/*
 * The three stages of the non-causal path, usable for causal attention too,
 * exposed with an explicit plan (chunk, segments) -- e.g. for a sequence
 * sharded over devices: each device
 * runs la_segment_states on its shard, the per-shard states are exchanged, and
 * la_segment_outputs runs from the exchanged prefix.
 *
 * ws layout (fp32): [B*H][segments + 1][D*M + D]; slot s of a head holds a state
 * (S row major [D][M], then z [D]).
 *
 * la_segment_states: slot s (s < nstates, nstates = segments or segments - 1)
 *   := sum over the positions of segment s of phi(k_j) v_j^T and phi(k_j).
 * la_segment_scan: turns slots 0..segments-1 into exclusive prefixes (slot s :=
 *   sum of the states of segments < s, in segment order) and writes the sum of
 *   all nstates states to slot `segments`; writes it to S_out/z_out if given
 *   (only meaningful when nstates == segments).
 * la_segment_outputs: out rows of segment s from slot s (causal) or from slot
 *   `segments` (non-causal); with causal = 1 and S_out/z_out given, the last
 *   segment also writes the final state.
 * ws_bytes must be at least (B*H) * (segments+1) * (D*M+D) * 4.
 */
LA_API int la_segment_states(const void *K, const void *V, float *ws, size_t ws_bytes,
                             int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                             int dtype, int chunk, int segments, int nstates, void *stream);
LA_API int la_segment_scan(float *ws, size_t ws_bytes, int64_t B, int64_t H, int64_t D, int64_t M,
                           int segments, int nstates, float *S_out, float *z_out, void *stream);
LA_API int la_segment_outputs(const void *Q, const void *K, const void *V, void *out,
                              const float *ws, size_t ws_bytes,
                              int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                              int causal, int dtype, int chunk, int segments,
                              float *S_out, float *z_out, void *stream);

/*
 * One recurrent (autoregressive) step for B*H independent heads (page
 * "Transformers are RNNs", Proposed method: the causal model as an RNN with
 * memories (S, z); Main findings: the state is updated incrementally).
 *   S += phi(k) v^T;  z += phi(k);  out = phi(q)^T S / (phi(q)^T z)
 * The token enters the state before the read-out, matching the causal mode's
 * j <= i.  S [B][H][D][M] and z [B][H][D] (fp32) are read and rewritten in place
 * (start from zeros for an empty history).  q, k: [B][H][D]; v: [B][H][M];
 * out: [B][H][M] fp32.  The state is the whole history: copying S and z out and
 * back resumes a sequence exactly.  D and M: any multiple of 16 up to 128.
 */
LA_API int la_decode_step(float *S, float *z, const void *q, const void *k, const void *v,
                          float *out, int64_t B, int64_t H, int64_t D, int64_t M,
                          int dtype, void *stream);

/*
 * Gradients of causal attention (training backward of the parallel mode; page
 * "Transformers are RNNs", Proposed method: gradients in linear time and
 * constant memory, by running sums like the forward pass).  For a loss L with
 * dout = dL/dout, with g = phi(q), f = phi(k), den_i = g_i . z_i:
 *   r_i = dout_i / den_i,  c_i = -(dout_i . out_i) / den_i
 *   dL/dq_i = (S_i r_i + c_i z_i) * phi'(q_i)            (sums over j <= i)
 *   dL/dk_j = (R_j v_j + w_j) * phi'(k_j),  dL/dv_j = R_j^T phi(k_j)
 * with R_j = sum_{i>=j} g_i r_i^T, w_j = sum_{i>=j} c_i g_i (sums over i >= j)
 * and phi'(x) = 1 for x > 0, exp(x) otherwise.
 * out: the forward's output [B][H][N][M] fp32 (from la_forward_chunked, causal);
 * dout [B][H][N][M] fp32; dQ, dK [B][H][N][D] and dV [B][H][N][M] fp32, fully
 * written.  Q, K, V as for the forward (fp32 or bf16); all arithmetic fp32.
 * dtype LA_F32_FEATURES: Q and K hold features phi(q), phi(k) (fp32, V fp32,
 * D the feature dimension); phi' is then 1, so dQ and dK are the gradients with
 * respect to those features (la_feature_map_backward carries them on to the
 * raw rows).  LA_OUT_BF16 is refused.
 * workspace: at least la_backward_workspace_bytes(...) bytes, no
 * initialisation needed (every byte the call reads it writes first).
 * Five kernels on `stream`: segment states, their scan, dQ (with the reverse
 * segment states), the reverse scan, dK and dV.
 */
LA_API size_t la_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                                          int dtype);
LA_API int la_backward_chunked(const void *Q, const void *K, const void *V, const float *out,
                               const float *dout, float *dQ, float *dK, float *dV,
                               int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * T consecutive recurrent steps of every head in one call (the state is read
 * once and written once; page "Transformers are RNNs", Proposed method: the
 * RNN update applied token after token).  Equivalent to T calls of
 * la_decode_step with q, k, v, out of token t, up to rounding.
 * q, k: [B][H][T][D]; v, out: [B][H][T][M]; S, z updated in place.
 * T = 0 is a valid empty call.  Same element types, alignment and status
 * codes as la_decode_step.  Short calls run the recurrence with the state in
 * registers; longer ones with fp32 inputs (12+ tokens for states of 4096+
 * values, 16+ for 2048+, 32+ for any, when every head is one segment of the
 * forward planner) run the chunked causal kernel continuing from S, z in place
 * (la_forward_continue's fp32 arithmetic on MFMA tiles), which is faster there.
 * Arithmetic is fp32 for both input types.
 */
LA_API int la_decode_steps(float *S, float *z, const void *q, const void *k, const void *v,
                           float *out, int64_t B, int64_t H, int64_t T, int64_t D, int64_t M,
                           int dtype, void *stream);

/*
 * Softmax attention as an RNN (page "Attention as an RNN", Proposed method:
 * attention's many-to-many RNN outputs computed with a parallel prefix scan;
 * the query is a learned vector).  One query q per head; with s_i = q . k_i (no
 * scaling -- scale q beforehand) every position k receives the softmax
 * attention of q over positions 0..k:
 *   out_k = sum_{i<=k} exp(s_i) v_i / sum_{i<=k} exp(s_i),
 * evaluated with the running state (m, u, w) = (max s, sum exp(s - m),
 * sum exp(s - m) v), which never overflows.
 * q: [B][H][D]; K: [B][H][N][D]; V: [B][H][N][M] (fp32 or bf16); out
 * [B][H][N][M] fp32.  m_out, u_out [B][H] and w_out [B][H][M] fp32: optional
 * (all or none), the state after the last position, for la_softmax_step.
 * workspace: la_softmax_scan_workspace_bytes(...) bytes (0 when every head fits
 * one group of 128 positions), zeroed (la_workspace_init)
 * before its first use, then reusable by later calls with the same shape;
 * calls sharing a workspace must not overlap.  Waits for earlier groups are
 * bounded as for la_forward_chunked (same error word and poll-cap word); a
 * wait that gives up leaves NaN in the affected outputs and final state.
 */
LA_API size_t la_softmax_scan_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M);
LA_API int la_softmax_scan(const void *q, const void *K, const void *V, float *out,
                           int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype,
                           void *workspace, size_t workspace_bytes,
                           float *m_out, float *u_out, float *w_out, void *stream);

/*
 * One token of the same RNN for every head, in constant memory: the state
 * m [B][H], u [B][H], w [B][H][M] (fp32, updated in place; a fresh state is
 * m = -inf, u = 0, w = 0) takes (k, v) and out receives the attention of q over
 * every token seen so far.  q, k [B][H][D]; v, out [B][H][M].
 */
LA_API int la_softmax_step(float *m, float *u, float *w, const void *q, const void *k,
                           const void *v, float *out, int64_t B, int64_t H, int64_t D,
                           int64_t M, int dtype, void *stream);

/* Random-feature map with feature dimension F (page "Stable, Fast and
 * Accurate: Kernelized Attention with Relative Positional Encoding", Proposed
 * method and Main findings: kernelized attention with the feature maps PRF,
 * TRF, Sphere-PRF and ORF, feature dimension as small as 16, queries and keys
 * normalised when their norms are large).  Each row x of X is mapped to F
 * features in out:
 *   LA_FEATURE_ELU: elu(x) + 1 elementwise (F = D; W unused, may be NULL);
 *   LA_FEATURE_PRF: exp(w_p . x - |x|^2 / 2) / sqrt(F), p < F, W [F][D] fp32;
 *   LA_FEATURE_TRF: with P = F / 2 and c = exp(|x|^2 / 2) / sqrt(P):
 *                   out[p] = c sin(w_p . x), out[P + p] = c cos(w_p . x),
 *                   W [P][D] fp32.
 * Over rows w_p ~ N(0, I) the expected phi(q) . phi(k) is exp(q . k) for PRF
 * and TRF.  ORF (orthogonal rows) and Sphere-PRF (rows on a sphere) are PRF
 * with the caller's W.  flags: LA_FEATURE_NORMALIZE scales every row to unit
 * length first (a zero row stays zero).
 * X [rows][D] (dtype LA_F32 or LA_BF16), out [rows][F] fp32.  X2 / out2: an
 * optional second tensor of the same shape mapped in the same launch (both NULL
 * or both set), e.g. Q and K.  D and F must each be 16, 32, 64 or 128.  The
 * outputs feed the other entry points with dtype LA_F32_FEATURES.
 */
enum la_feature_kind { LA_FEATURE_ELU = 0, LA_FEATURE_PRF = 1, LA_FEATURE_TRF = 2 };
enum { LA_FEATURE_NORMALIZE = 1 };
LA_API int la_feature_map(float *out, const void *X, float *out2, const void *X2, int64_t rows, int64_t D,
                          int dtype, const float *W, int64_t F, int kind, int flags, void *stream);

/* Gradient of la_feature_map with respect to its input rows: dX = J(x)^T dOut
 * for every row x of X, where J is the Jacobian of the map (same X, dtype, W, F,
 * kind and flags as the forward call).  By the chain rule through the
 * definitions above (page "Stable, Fast and Accurate: Kernelized Attention with
 * Relative Positional Encoding", Proposed method): for PRF
 * d phi_p / dx = phi_p (w_p - x); for TRF the magnitude c contributes c x and
 * the angle c cos / -c sin times w_p; elu: 1 for x > 0, exp(x) otherwise; with
 * LA_FEATURE_NORMALIZE the unit-length scaling contributes (I - y y^T) / |x|
 * (y = x / |x|), and a zero row gets a zero gradient.  dOut [rows][F] fp32,
 * dX [rows][D] fp32 (4-byte alignment suffices).  Together with
 * la_backward_chunked on LA_F32_FEATURES inputs (the gradients with respect to
 * the features) this gives the gradients of attention through a random-feature
 * map.  D and F as for la_feature_map.
 */
LA_API int la_feature_map_backward(float *dX, const void *X, const float *dOut, int64_t rows, int64_t D, int dtype,
                                   const float *W, int64_t F, int kind, int flags, void *stream);

/* One recurrent step (as la_decode_step) on raw rows with the random-feature
 * map formed inside the kernel: q, k [B][H][D] raw rows and v [B][H][M], all of
 * element type dtype (LA_F32 or LA_BF16, widened exactly); W, F, kind (PRF or
 * TRF) and flags (LA_FEATURE_NORMALIZE) as for la_feature_map; S [B][H][F][M]
 * and z [B][H][F] fp32, updated in place (the state la_forward_features leaves
 * in S_out, z_out); out [B][H][M] fp32.  F must be 16, 32 or 64.  Equals
 * la_feature_map followed by la_decode_step with LA_F32_FEATURES.
 */
LA_API int la_decode_step_features(float *S, float *z, const void *q, const void *k, const void *v, float *out,
                                   int64_t B, int64_t H, int64_t D, int64_t M, int dtype, const float *W, int64_t F,
                                   int kind, int flags, void *stream);

/* Attention on random features of raw rows in one call: each chunk's raw q, k
 * rows are mapped to F features (as la_feature_map, kinds LA_FEATURE_PRF and
 * LA_FEATURE_TRF, flag LA_FEATURE_NORMALIZE) and attended to as with
 * la_forward_chunked on LA_F32_FEATURES inputs.  On one-pass plans the map is
 * fused into the attention kernel's staging and the features never reach
 * memory (other plans: see Plan below).  causal = 1 or 0 as for
 * la_forward_chunked (0: the stage kernels, the map in both; no states).
 * Q, K [B][H][N][D] (raw rows) and V [B][H][N][M], all of element type dtype
 * (LA_F32 or LA_BF16; bf16 values are widened exactly, the map and the
 * attention run in fp32 as for fp32 rows), W as for la_feature_map, out
 * [B][H][N][M] fp32; S_in [B][H][F][M], z_in [B][H][F] optional (both or
 * neither): a carried state the sequence continues from (as for
 * la_forward_continue; S_out may be S_in for an in-place update, so a call on T
 * new tokens is a T-token decode step); S_out [B][H][F][M], z_out [B][H][F]
 * optional (both or neither): the final state over the features (causal = 1
 * only; with causal = 0 all four must be NULL).
 * workspace: la_forward_features_workspace_bytes(...) bytes (at least 256 for
 * a supported shape, 0 for a refused one), initialised and reused as for
 * la_forward_chunked.
 * Plan: chunks of 32, segments sized for 512 resident workgroups; causal: the
 * one-pass kernel runs segments of at most four chunks where its LDS fits;
 * everything else runs as two launches, the map into the workspace and then the
 * attention kernels on those features (bf16 V widened into the workspace), which
 * measured faster there than a fused two-phase kernel (that forms the k-row
 * projections in both of its phases).  The features then pass through memory
 * (rows * F * 8 bytes of workspace, plus rows * M * 4 for V).  D and F
 * outside the supported set (D, F and M in {16, 32, 64, 128}; non-causal F up
 * to 64) give LA_ERR_UNSUPPORTED (and a workspace size of 0); F = 128 always runs
 * as two launches.
 */
LA_API size_t la_forward_features_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int64_t F,
                                                  int causal);
LA_API int la_forward_features(const void *Q, const void *K, const void *V, float *out, int64_t B, int64_t H,
                               int64_t N, int64_t D, int64_t M, int causal, int dtype, const float *W, int64_t F,
                               int kind, int flags, void *workspace, size_t workspace_bytes, const float *S_in,
                               const float *z_in, float *S_out, float *z_out, void *stream);

/*
 * Peak probes (measurement support, not a step of the method): the attainable
 * rates that the kernels' rooflines are set against, beside the nominal peaks.
 *
 * la_probe_copy: copies `bytes` bytes from src to dst (device memory, both
 * 16-byte aligned, not overlapping; bytes a multiple of 16, else
 * LA_ERR_INVALID_ARG; 0 is a no-op).  Result bit-exact.  Read + written bytes
 * over the launch's time give the attainable HBM rate.
 *
 * la_probe_mfma: `blocks` workgroups of 256 threads (4 wavefronts); every
 * wavefront runs `iters` rounds of 8 independent MFMA chains: fp32 16x16x4
 * (dtype LA_F32, 2048 flops each) or bf16 16x16x32 (LA_BF16, 16384 flops each),
 * every operand element x (rounded to bf16 for LA_BF16).  Flops per launch:
 * blocks * 4 * iters * 8 * (2048 or 16384).  out [blocks * 256] fp32 (device):
 * lane i writes the sum of its 32 accumulator values, 32 * iters * K * x^2 with
 * K = 4 (fp32) or 32 (bf16), exact while that and iters * K * x^2 are integers
 * below 2^24.  blocks in [0, 2^20] and iters >= 0, else LA_ERR_INVALID_ARG;
 * blocks = 0 is a no-op.
 */
LA_API int la_probe_copy(void *dst, const void *src, size_t bytes, void *stream);
/* la_probe_read: sums the fp32 words of src (bytes % 16 == 0; 16-byte aligned)
 * with nontemporal 16-byte loads over a fixed grid; out receives one partial
 * sum per thread, la_probe_read_partials() floats in all (every one written,
 * also for bytes == 0).  Their sum is the sum of src up to rounding order (exact
 * for small integer values).  Measures the attainable read-only HBM rate. */
LA_API size_t la_probe_read_partials(void);
LA_API int la_probe_read(float *out, const void *src, size_t bytes, void *stream);
LA_API int la_probe_mfma(float *out, int dtype, int64_t blocks, int iters, float x, void *stream);
/* la_probe_write: fills `bytes` bytes of dst (device memory, 16-byte aligned;
 * bytes a multiple of 16, else LA_ERR_INVALID_ARG; 0 is a no-op) with the fp32
 * value `value` by nontemporal 16-byte stores.  Result bit-exact.  Written bytes
 * over the launch's time give the attainable write-only HBM rate. */
LA_API int la_probe_write(void *dst, size_t bytes, float value, void *stream);
/* la_probe_mfma32: as la_probe_mfma with LA_BF16, on the bf16 32x32x16 shape:
 * every wavefront runs `iters` rounds of 4 independent chains (32768 flops per
 * MFMA), so flops per launch = blocks * 4 * iters * 4 * 32768; lane i writes the
 * sum of its 64 accumulator values, 64 * iters * 16 * x^2 (x rounded to bf16),
 * exact while that is an integer below 2^24.  blocks in [0, 2^20] and iters >= 0,
 * else LA_ERR_INVALID_ARG; blocks = 0 is a no-op. */
LA_API int la_probe_mfma32(float *out, int64_t blocks, int iters, float x, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
