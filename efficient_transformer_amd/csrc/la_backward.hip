// Backward kernels instantiated for D, M in {16, 32, 64, 128}: fp32 and bf16 inputs
// through phi = elu + 1 (dtype 0, 1), fp32 inputs that already hold features (dtype 2).
#include "la_backward.hpp"
#include "la_launch.hpp"

namespace la {

hipError_t backward_dq(int dtype, int D, int M, const void *Q, const void *K, const void *V, const float *O,
                       const float *dO, const float *fwd_ws, float *rev_ws, float *den, float *dQ, int BH, int N,
                       int G, int CPS, hipStream_t stream) {
#define X(D_, M_)                                                                                             \
    if (D == D_ && M == M_)                                                                                   \
        return dtype == 0   ? run_bwd_dq<float, D_, M_>(Q, K, V, O, dO, fwd_ws, rev_ws, den, dQ, BH, N, G, CPS, stream) \
               : dtype == 2 ? run_bwd_dq<float, D_, M_, false>(Q, K, V, O, dO, fwd_ws, rev_ws, den, dQ, BH, N, G, CPS,  \
                                                              stream)                                                  \
                            : run_bwd_dq<bf16, D_, M_>(Q, K, V, O, dO, fwd_ws, rev_ws, den, dQ, BH, N, G, CPS, stream);
#define XM(D_) X(D_, 16) X(D_, 32) X(D_, 64) X(D_, 128)
    XM(16) XM(32) XM(64) XM(128)
#undef XM
#undef X
    return hipErrorInvalidValue;
}

hipError_t backward_dkv(int dtype, int D, int M, const void *Q, const void *K, const void *V, const float *O,
                        const float *dO, const float *rev_ws, const float *den, float *dK, float *dV, int BH, int N,
                        int G, int CPS, hipStream_t stream) {
#define X(D_, M_)                                                                                            \
    if (D == D_ && M == M_)                                                                                  \
        return dtype == 0   ? run_bwd_dkv<float, D_, M_>(Q, K, V, O, dO, rev_ws, den, dK, dV, BH, N, G, CPS, stream) \
               : dtype == 2 ? run_bwd_dkv<float, D_, M_, false>(Q, K, V, O, dO, rev_ws, den, dK, dV, BH, N, G, CPS,  \
                                                               stream)                                              \
                            : run_bwd_dkv<bf16, D_, M_>(Q, K, V, O, dO, rev_ws, den, dK, dV, BH, N, G, CPS, stream);
#define XM(D_) X(D_, 16) X(D_, 32) X(D_, 64) X(D_, 128)
    XM(16) XM(32) XM(64) XM(128)
#undef XM
#undef X
    return hipErrorInvalidValue;
}

hipError_t backward_rev_scan(float *ws, int BH, int E, int G, hipStream_t stream) {
    if (BH <= 0 || G <= 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_rev_scan_kernel, dim3((unsigned)((E + 255) / 256), (unsigned)BH), dim3(256), 0, stream, ws,
                       E, G);
    return hipGetLastError();
}

}  // namespace la
