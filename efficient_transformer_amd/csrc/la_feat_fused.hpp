// The one-pass causal kernel with the random-feature map fused into the staging
// of Q and K, dispatched over the raw-row width DI (16, 32, 64, 128), the
// feature count F (16, 32, 64) and M (16, 32, 64, 128); chunk 32.  TI is the
// element type of the raw rows and of V (fp32 or bf16).
#pragma once

#include "la_launch.hpp"
#include "la_prefill.hpp"

namespace la {

// The one-pass kernel (segments of at most four chunks); longer segments run the
// map and the attention as two launches (la_forward_features).
template <typename TI>
hipError_t prefill_features_typed(int DI, int F, int M, const void *Q, const void *K, const void *V, const float *W,
                                  int kind, int norm, float *out, void *ws, int BH, int N, int G, int CPS,
                                  float *S_out, float *z_out, const float *S_in, const float *z_in,
                                  hipStream_t stream) {
#define X(DI_, F_, M_)                                                                                          \
    if (DI == DI_ && F == F_ && M == M_)                                                                        \
        return run_onepass_features<DI_, F_, M_, kFusedFeatureChunk, TI>(Q, K, V, W, kind, norm, out, ws, BH, N, G, \
                                                                         CPS, S_out, z_out, S_in, z_in, stream);
#define XM(DI_, F_) X(DI_, F_, 16) X(DI_, F_, 32) X(DI_, F_, 64) X(DI_, F_, 128)
#define XF(DI_) XM(DI_, 16) XM(DI_, 32) XM(DI_, 64)
    XF(16) XF(32) XF(64) XF(128)
#undef XF
#undef XM
#undef X
    return hipErrorInvalidValue;
}

// Non-causal: the stage path with the map in both stage kernels.
template <typename TI>
hipError_t prefill_features_noncausal_typed(int DI, int F, int M, const void *Q, const void *K, const void *V,
                                            const float *W, int kind, int norm, float *out, float *ws, int BH, int N,
                                            int G, int CPS, hipStream_t stream) {
#define X(DI_, F_, M_)                                                                                           \
    if (DI == DI_ && F == F_ && M == M_)                                                                         \
        return run_noncausal_features<DI_, F_, M_, kFusedFeatureChunk, TI>(Q, K, V, W, kind, norm, out, ws, BH, N, \
                                                                           G, CPS, stream);
#define XM(DI_, F_) X(DI_, F_, 16) X(DI_, F_, 32) X(DI_, F_, 64) X(DI_, F_, 128)
#define XF(DI_) XM(DI_, 16) XM(DI_, 32) XM(DI_, 64)
    XF(16) XF(32) XF(64) XF(128)
#undef XF
#undef XM
#undef X
    return hipErrorInvalidValue;
}

}  // namespace la
