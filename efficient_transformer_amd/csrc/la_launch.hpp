// Host-side launchers behind the C ABI (internal; not part of the public header).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace la {

// Element types of the inputs: fp32, bf16, or fp32 rows that already hold the
// features phi(q), phi(k) (the kernels then apply no feature map).
constexpr int kDtypeF32 = 0, kDtypeBf16 = 1, kDtypeF32Features = 2;
// OR-ed into the element type of bf16 inputs: the prefill outputs are bf16.
constexpr int kOutBf16 = 16;

// Workspace layout of the fused causal kernel (shared by host sizing and device code):
// header words, then one flag word per segment (padded to 64 words), then the
// aggregate and the inclusive state of every segment (E floats each).
constexpr int kWsHeaderWords = 64;
// header words of a look-back workspace: 1 heads counted, 2 epoch, 3 error
// (a wait gave up), 4 poll cap (0: the built-in bound; set by tests only)
constexpr int kWsErrorWord = 3;
constexpr int kWsPollCapWord = 4;
__host__ __device__ inline size_t fused_flag_words(long BHG) { return ((size_t)BHG + 63) / 64 * 64; }
// floats of one exchanged state slot: E = D*M + D padded to whole 256-byte blocks
__host__ __device__ inline int fused_slot_floats(int E) { return (E + 63) / 64 * 64; }
__host__ __device__ inline size_t fused_ws_bytes(long BH, int G, int E) {
    const size_t BHG = (size_t)BH * (size_t)G;
    return (kWsHeaderWords + fused_flag_words((long)BHG)) * 4 + 2 * BHG * (size_t)fused_slot_floats(E) * 4;
}

// Softmax scan (la_softmax_scan.hip): one state = M value sums + max + sum,
// padded to whole 256-byte blocks; workspace = header + flags + 2 states per
// group of softmax_scan_rows(M) rows.
__host__ __device__ constexpr int scan_slot_floats(int M) { return (M + 2 + 63) / 64 * 64; }
__host__ __device__ inline size_t scan_ws_bytes(long items, int M) {
    return (kWsHeaderWords + fused_flag_words(items)) * 4 + 2 * (size_t)items * (size_t)scan_slot_floats(M) * 4;
}
int softmax_scan_rows(int M);
hipError_t softmax_scan(int dtype, int D, int M, const void *q, const void *K, const void *V, float *out, void *ws,
                        int BH, int N, float *m_out, float *u_out, float *w_out, hipStream_t stream);
hipError_t softmax_step(int dtype, int D, int M, float *m, float *u, float *w, const void *q, const void *k,
                        const void *v, float *out, int BH, hipStream_t stream);

// Prefill stage launchers for one element type (kDtype*).
// Each returns hipErrorInvalidValue for a (D, M, C) combination that has no kernel.
bool prefill_supported(int dtype, int D, int M, int C);
hipError_t prefill_states(int dtype, int D, int M, int C, const void *K, const void *V, float *ws, int BH, int N,
                          int G, int CPS, int nstates, hipStream_t stream);
hipError_t prefill_outputs(int dtype, int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                           const float *ws, int BH, int N, int G, int CPS, int causal, float *S_out, float *z_out,
                           hipStream_t stream);
hipError_t prefill_fused(int dtype, int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                         void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in, const float *z_in, hipStream_t stream);
// One-pass causal kernel: segments of at most 4 chunks (see la_prefill.hpp).
constexpr int kOnePassMaxChunks = 4;
bool prefill_onepass_supported(int dtype, int D, int M, int C);
hipError_t prefill_onepass(int dtype, int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                           void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in, const float *z_in, hipStream_t stream);
size_t prefill_lds_bytes(int dtype, int D, int M, int C);
hipError_t prefill_scan(float *ws, int BH, int D, int M, int G, int nstates, float *S_out, float *z_out,
                        hipStream_t stream);
hipError_t fill_zero(float *p, size_t n, hipStream_t stream);

// Backward (la_backward.hip): chunk of 32 positions, stage workspaces as the forward's.
constexpr int kBackwardChunk = 32;
hipError_t backward_dq(int dtype, int D, int M, const void *Q, const void *K, const void *V, const float *O,
                       const float *dO, const float *fwd_ws, float *rev_ws, float *den, float *dQ, int BH, int N,
                       int G, int CPS, hipStream_t stream);
hipError_t backward_dkv(int dtype, int D, int M, const void *Q, const void *K, const void *V, const float *O,
                        const float *dO, const float *rev_ws, const float *den, float *dK, float *dV, int BH, int N,
                        int G, int CPS, hipStream_t stream);
hipError_t backward_rev_scan(float *ws, int BH, int E, int G, hipStream_t stream);

// one recurrent step on raw q, k rows (DI wide, fp32 or bf16) mapped to F random features in the kernel
hipError_t decode_step_features(int dtype, int DI, int F, int M, float *S, float *z, const void *q, const void *k,
                                const void *v, float *out, const float *W, int kind, int norm, int BH,
                                hipStream_t stream);
hipError_t decode_step(int dtype, int D, int M, float *S, float *z, const void *q, const void *k, const void *v,
                       float *out, int BH, hipStream_t stream);
hipError_t decode_steps(int dtype, int D, int M, float *S, float *z, const void *q, const void *k, const void *v,
                        float *out, int BH, int Tn, hipStream_t stream);

// Widths that are multiples of 16 up to 128 without a specialised kernel (la_pad.hip).
// pad_copy: dst[h][r][c] = src[h][r][c] for r < Rs and byte column c < Cs_bytes, else
// `fill` in every 32-bit word (rows of Cd_bytes, Rd rows per h); unpad_copy: the
// inverse selection.  Column widths are whole 16-byte units.
hipError_t pad_copy(const void *src, void *dst, long BH, long Rs, long Cs_bytes, long Rd, long Cd_bytes,
                    unsigned fill, hipStream_t stream);
hipError_t unpad_copy(const void *src, void *dst, long BH, long Rs, long Cs_bytes, long Rd, long Cd_bytes,
                      hipStream_t stream);
// n bf16 values (n % 8 == 0, 16-byte aligned) widened exactly to fp32.
hipError_t widen_bf16(const void *src, float *dst, long n, hipStream_t stream);
// Tn recurrent steps of every head for D, M given at run time (multiples of 16 up to 128).
hipError_t decode_any(int dtype, int D, int M, float *S, float *z, const void *q, const void *k, const void *v,
                      float *out, int BH, int Tn, hipStream_t stream);

// Random-feature map (la_features.hip): kind 0 elu (F = D), 1 positive, 2
// trigonometric; X2 / out2 optional (a second tensor in the same launch).
hipError_t feature_map(int dtype, int D, int F, int kind, const void *X, float *out, const void *X2, float *out2,
                       const float *W, long rows, bool norm, hipStream_t stream);
// Its gradient with respect to the rows of X: dX [rows][D] fp32 from dOut [rows][F].
hipError_t feature_map_backward(int dtype, int D, int F, int kind, const void *X, const float *dOut, const float *W,
                                float *dX, long rows, bool norm, hipStream_t stream);

// bf16 inputs, bf16 outputs (la_bf16out.hip)
hipError_t prefill_fused_bf16o(int D, int M, int C, const void *Q, const void *K, const void *V, void *out, void *ws,
                               int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in,
                               const float *z_in, hipStream_t stream);
hipError_t prefill_onepass_bf16o(int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                                 void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out,
                                 const float *S_in, const float *z_in, hipStream_t stream);
hipError_t prefill_outputs_bf16o(int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                                 const float *ws, int BH, int N, int G, int CPS, int causal, float *S_out,
                                 float *z_out, hipStream_t stream);

// random features fused into the one-pass causal kernel (la_feat_fused*.hip):
// raw rows (and V) fp32 or bf16, features and attention fp32
constexpr int kFusedFeatureChunk = 32;
// whether the one-pass kernel with the map fused fits (LDS) for this shape
bool prefill_features_onepass_supported(int DI, int F, int M);
// non-causal attention over random features (stage path; ws as la_segment_states')
bool prefill_features_noncausal_supported(int DI, int F, int M);
hipError_t prefill_features_noncausal(int dtype, int DI, int F, int M, const void *Q, const void *K, const void *V,
                                      const float *W, int kind, int norm, float *out, float *ws, int BH, int N, int G,
                                      int CPS, hipStream_t stream);
hipError_t prefill_features_noncausal_bf16(int DI, int F, int M, const void *Q, const void *K, const void *V,
                                           const float *W, int kind, int norm, float *out, float *ws, int BH, int N,
                                           int G, int CPS, hipStream_t stream);
hipError_t prefill_features_f32(int DI, int F, int M, const void *Q, const void *K, const void *V, const float *W,
                                int kind, int norm, float *out, void *ws, int BH, int N, int G, int CPS,
                                float *S_out, float *z_out, const float *S_in, const float *z_in,
                                hipStream_t stream);
hipError_t prefill_features_bf16(int DI, int F, int M, const void *Q, const void *K, const void *V, const float *W,
                                 int kind, int norm, float *out, void *ws, int BH, int N, int G, int CPS,
                                 float *S_out, float *z_out, const float *S_in, const float *z_in,
                                 hipStream_t stream);

// feature inputs (la_feat_prefill.hip, la_feat_onepass.hip)
bool prefill_supported_feat(int D, int M, int C);
size_t prefill_lds_bytes_feat(int D, int M, int C);
bool prefill_onepass_supported_feat(int D, int M, int C);
hipError_t prefill_states_feat(int D, int M, int C, const void *K, const void *V, float *ws, int BH, int N, int G,
                               int CPS, int nstates, hipStream_t stream);
hipError_t prefill_fused_feat(int D, int M, int C, const void *Q, const void *K, const void *V, float *out, void *ws,
                              int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in,
                              const float *z_in, hipStream_t stream);
hipError_t prefill_outputs_feat(int D, int M, int C, const void *Q, const void *K, const void *V, float *out,
                                const float *ws, int BH, int N, int G, int CPS, int causal, float *S_out,
                                float *z_out, hipStream_t stream);
hipError_t prefill_onepass_feat(int D, int M, int C, const void *Q, const void *K, const void *V, float *out,
                                void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out,
                                const float *S_in, const float *z_in, hipStream_t stream);

// per element type (defined in la_prefill_f32.hip / la_prefill_bf16.hip)
hipError_t prefill_fused_f32(int D, int M, int C, const void *Q, const void *K, const void *V, float *out, void *ws,
                             int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in, const float *z_in, hipStream_t stream);
hipError_t prefill_fused_bf16(int D, int M, int C, const void *Q, const void *K, const void *V, float *out, void *ws,
                              int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in, const float *z_in, hipStream_t stream);
hipError_t prefill_onepass_f32(int D, int M, int C, const void *Q, const void *K, const void *V, float *out,
                               void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in, const float *z_in, hipStream_t stream);
hipError_t prefill_onepass_bf16(int D, int M, int C, const void *Q, const void *K, const void *V, float *out,
                                void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out,
                                const float *S_in, const float *z_in,
                                hipStream_t stream);
bool prefill_onepass_supported_f32(int D, int M, int C);
bool prefill_onepass_supported_bf16(int D, int M, int C);
size_t prefill_lds_bytes_f32(int D, int M, int C);
size_t prefill_lds_bytes_bf16(int D, int M, int C);
bool prefill_supported_f32(int D, int M, int C);
bool prefill_supported_bf16(int D, int M, int C);
hipError_t prefill_states_f32(int D, int M, int C, const void *K, const void *V, float *ws, int BH, int N, int G,
                              int CPS, int nstates, hipStream_t stream);
hipError_t prefill_states_bf16(int D, int M, int C, const void *K, const void *V, float *ws, int BH, int N, int G,
                               int CPS, int nstates, hipStream_t stream);
hipError_t prefill_outputs_f32(int D, int M, int C, const void *Q, const void *K, const void *V, float *out,
                               const float *ws, int BH, int N, int G, int CPS, int causal, float *S_out,
                               float *z_out, hipStream_t stream);
hipError_t prefill_outputs_bf16(int D, int M, int C, const void *Q, const void *K, const void *V, float *out,
                                const float *ws, int BH, int N, int G, int CPS, int causal, float *S_out,
                                float *z_out, hipStream_t stream);

}  // namespace la
