// Prefill kernels for inputs that already hold features (fp32 phi(Q), phi(K), for
// example from the random-feature map): the same kernels as for fp32 inputs with
// the feature map switched off.  D (the feature dimension), M in {16, 32, 64, 128},
// C in {16, 32, 64}.
#include "la_launch.hpp"
#include "la_prefill.hpp"

namespace la {

bool prefill_supported_feat(int D, int M, int C) { return prefill_supported_f32(D, M, C); }
size_t prefill_lds_bytes_feat(int D, int M, int C) { return prefill_lds_bytes_f32(D, M, C); }
bool prefill_onepass_supported_feat(int D, int M, int C) { return prefill_onepass_supported_f32(D, M, C); }

hipError_t prefill_states_feat(int D, int M, int C, const void *K, const void *V, float *ws, int BH, int N, int G,
                               int CPS, int nstates, hipStream_t stream) {
#define X(D_, M_, C_) \
    if (D == D_ && M == M_ && C == C_) \
        return run_states<float, D_, M_, C_, false>(K, V, ws, BH, N, G, CPS, nstates, stream);
    LA_FOR_ALL(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t prefill_fused_feat(int D, int M, int C, const void *Q, const void *K, const void *V, float *out, void *ws,
                              int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in,
                              const float *z_in, hipStream_t stream) {
#define X(D_, M_, C_) \
    if (D == D_ && M == M_ && C == C_) \
        return run_fused<float, D_, M_, C_, false>(Q, K, V, out, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream);
    LA_FOR_ALL(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t prefill_outputs_feat(int D, int M, int C, const void *Q, const void *K, const void *V, float *out,
                                const float *ws, int BH, int N, int G, int CPS, int causal, float *S_out,
                                float *z_out, hipStream_t stream) {
#define X(D_, M_, C_) \
    if (D == D_ && M == M_ && C == C_) \
        return run_outputs<float, D_, M_, C_, false>(Q, K, V, out, ws, BH, N, G, CPS, causal, S_out, z_out, stream);
    LA_FOR_ALL(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace la
