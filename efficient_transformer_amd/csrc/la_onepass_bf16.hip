// One-pass causal prefill kernels instantiated for bf16 inputs: D, M in {16, 32, 64, 128}, C in {16, 32, 64}.
#include "la_launch.hpp"
#include "la_prefill.hpp"

namespace la {

static_assert(kOnePassChunks == kOnePassMaxChunks, "one-pass segment bound");

bool prefill_onepass_supported_bf16(int D, int M, int C) {
#define X(D_, M_, C_) \
    if (D == D_ && M == M_ && C == C_) return Cfg<bf16, D_, M_, C_>::fits && OnePassLds<bf16, D_, M_, C_>::fits;
    LA_FOR_ALL(X)
#undef X
    return false;
}

hipError_t prefill_onepass_bf16(int D, int M, int C, const void *Q, const void *K, const void *V, float *out, void *ws,
                             int BH, int N, int G, int CPS, float *S_out, float *z_out, const float *S_in,
                             const float *z_in, hipStream_t stream) {
#define X(D_, M_, C_) \
    if (D == D_ && M == M_ && C == C_) \
        return run_onepass<bf16, D_, M_, C_>(Q, K, V, out, ws, BH, N, G, CPS, S_out, z_out, S_in, z_in, stream);
    LA_FOR_ALL(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace la
