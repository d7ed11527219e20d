// Prefill kernels for bf16 inputs that write bf16 outputs (rounded to nearest
// even from the fp32 result): the two causal kernels and the stage read-out.
// D, M in {16, 32, 64, 128}, C in {16, 32, 64}.
#include "la_launch.hpp"
#include "la_prefill.hpp"

namespace la {

hipError_t prefill_fused_bf16o(int D, int M, int C, const void *Q, const void *K, const void *V, void *out, void *ws,
                               int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in,
                               const float *z_in, hipStream_t stream) {
#define X(D_, M_, C_) \
    if (D == D_ && M == M_ && C == C_) \
        return run_fused<bf16, D_, M_, C_, true, bf16>(Q, K, V, out, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, \
                                                       stream);
    LA_FOR_ALL(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t prefill_onepass_bf16o(int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                                 void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out,
                                 const float *S_in, const float *z_in, hipStream_t stream) {
#define X(D_, M_, C_) \
    if (D == D_ && M == M_ && C == C_) \
        return run_onepass<bf16, D_, M_, C_, true, bf16>(Q, K, V, out, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, \
                                                         stream);
    LA_FOR_ALL(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t prefill_outputs_bf16o(int D, int M, int C, const void *Q, const void *K, const void *V, void *out,
                                 const float *ws, int BH, int N, int G, int CPS, int causal, float *S_out,
                                 float *z_out, hipStream_t stream) {
#define X(D_, M_, C_) \
    if (D == D_ && M == M_ && C == C_) \
        return run_outputs<bf16, D_, M_, C_, true, bf16>(Q, K, V, out, ws, BH, N, G, CPS, causal, S_out, z_out, \
                                                         stream);
    LA_FOR_ALL(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace la
