// One-pass causal prefill kernels for inputs that already hold features (fp32,
// the feature map switched off): D (the feature dimension), M in
// {16, 32, 64, 128}, C in {16, 32, 64}.
#include "la_launch.hpp"
#include "la_prefill.hpp"

namespace la {

hipError_t prefill_onepass_feat(int D, int M, int C, const void *Q, const void *K, const void *V, float *out,
                                void *ws, int BH, int N, int G, int CPS, float *S_out, float *z_out,
                                const float *S_in, const float *z_in, hipStream_t stream) {
#define X(D_, M_, C_) \
    if (D == D_ && M == M_ && C == C_) \
        return run_onepass<float, D_, M_, C_, false>(Q, K, V, out, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, \
                                                     stream);
    LA_FOR_ALL(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace la
