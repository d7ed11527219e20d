// Fused random features, bf16 raw rows (mapped and attended to in fp32).
#include "la_feat_fused.hpp"

namespace la {

hipError_t prefill_features_bf16(int DI, int F, int M, const void *Q, const void *K, const void *V, const float *W,
                                 int kind, int norm, float *out, void *ws, int BH, int N, int G, int CPS,
                                 float *S_out, float *z_out, const float *S_in, const float *z_in,
                                 hipStream_t stream) {
    return prefill_features_typed<bf16>(DI, F, M, Q, K, V, W, kind, norm, out, ws, BH, N, G, CPS, S_out, z_out, S_in,
                                        z_in, stream);
}

hipError_t prefill_features_noncausal_bf16(int DI, int F, int M, const void *Q, const void *K, const void *V,
                                           const float *W, int kind, int norm, float *out, float *ws, int BH, int N,
                                           int G, int CPS, hipStream_t stream) {
    return prefill_features_noncausal_typed<bf16>(DI, F, M, Q, K, V, W, kind, norm, out, ws, BH, N, G, CPS, stream);
}

}  // namespace la
