// Fused random features, fp32 raw rows (and the shape check shared by both types).
#include "la_feat_fused.hpp"

namespace la {

bool prefill_features_noncausal_supported(int DI, int F, int M) {
#define X(DI_, F_, M_) \
    if (DI == DI_ && F == F_ && M == M_) return stage_features_fit<DI_, F_, M_, kFusedFeatureChunk>();
#define XM(DI_, F_) X(DI_, F_, 16) X(DI_, F_, 32) X(DI_, F_, 64) X(DI_, F_, 128)
#define XF(DI_) XM(DI_, 16) XM(DI_, 32) XM(DI_, 64)
    XF(16) XF(32) XF(64) XF(128)
#undef XF
#undef XM
#undef X
    return false;
}

hipError_t prefill_features_noncausal(int dtype, int DI, int F, int M, const void *Q, const void *K, const void *V,
                                      const float *W, int kind, int norm, float *out, float *ws, int BH, int N, int G,
                                      int CPS, hipStream_t stream) {
    return dtype == kDtypeF32 ? prefill_features_noncausal_typed<float>(DI, F, M, Q, K, V, W, kind, norm, out, ws, BH,
                                                                         N, G, CPS, stream)
                              : prefill_features_noncausal_bf16(DI, F, M, Q, K, V, W, kind, norm, out, ws, BH, N, G,
                                                                CPS, stream);
}

bool prefill_features_onepass_supported(int DI, int F, int M) {
#define X(DI_, F_, M_) \
    if (DI == DI_ && F == F_ && M == M_) return onepass_features_fit<DI_, F_, M_, kFusedFeatureChunk>();
#define XM(DI_, F_) X(DI_, F_, 16) X(DI_, F_, 32) X(DI_, F_, 64) X(DI_, F_, 128)
#define XF(DI_) XM(DI_, 16) XM(DI_, 32) XM(DI_, 64)
    XF(16) XF(32) XF(64) XF(128)
#undef XF
#undef XM
#undef X
    return false;
}

hipError_t prefill_features_f32(int DI, int F, int M, const void *Q, const void *K, const void *V, const float *W,
                                int kind, int norm, float *out, void *ws, int BH, int N, int G, int CPS,
                                float *S_out, float *z_out, const float *S_in, const float *z_in,
                                hipStream_t stream) {
    return prefill_features_typed<float>(DI, F, M, Q, K, V, W, kind, norm, out, ws, BH, N, G, CPS, S_out, z_out, S_in,
                                         z_in, stream);
}

}  // namespace la
