/* Host sanitizer run of the C ABI's argument validation and planning (test
 * infrastructure only).  Every call here is answered by the library's checks or
 * its planner before any HIP runtime call, so no GPU is needed; the library's
 * host code is built with AddressSanitizer and UndefinedBehaviorSanitizer. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "linattn.h"

static int fails = 0;
#define EXPECT(cond, what)                          \
    do {                                            \
        if (!(cond)) {                              \
            fprintf(stderr, "FAIL %s\n", what);     \
            ++fails;                                \
        }                                           \
    } while (0)

int main(void) {
    void *const F = (void *)(uintptr_t)0x10000; /* aligned, never dereferenced */
    for (int s = -1; s <= 6; ++s) EXPECT(la_status_str(s) != NULL && strlen(la_status_str(s)) > 0, "status string");
    EXPECT(la_version() >= 100, "version");
    /* plans over widths, chunks, dtypes and sizes, including padded widths and extremes */
    const int64_t widths[] = {16, 32, 48, 64, 80, 96, 112, 128, 8, 40, 144, 0, -16};
    const int dtypes[] = {LA_F32, LA_BF16, LA_F32_FEATURES, LA_BF16 | LA_OUT_BF16, 3, -1};
    const int chunks[] = {0, 16, 32, 64, 128, 7};
    const int64_t Ns[] = {0, 1, 63, 64, 65, 1000, 65536, (int64_t)1 << 31, -1};
    for (unsigned a = 0; a < sizeof widths / sizeof *widths; ++a)
        for (unsigned b = 0; b < sizeof widths / sizeof *widths; b += 3)
            for (unsigned t = 0; t < sizeof dtypes / sizeof *dtypes; ++t)
                for (unsigned c = 0; c < sizeof chunks / sizeof *chunks; ++c)
                    for (unsigned n = 0; n < sizeof Ns / sizeof *Ns; ++n)
                        for (int causal = 0; causal <= 2; ++causal) {
                            int ch = -1, seg = -1;
                            size_t ws = 0;
                            const int64_t D = widths[a], M = widths[b];
                            int st = la_forward_plan(2, 3, Ns[n], D, M, causal, dtypes[t], chunks[c], &ch, &seg, &ws);
                            size_t ws2 = la_forward_workspace_bytes(2, 3, Ns[n], D, M, causal, dtypes[t], chunks[c]);
                            EXPECT(st == LA_OK ? ws2 == ws : ws2 == 0, "plan and workspace bytes agree");
                            if (st == LA_OK && Ns[n] > 0) EXPECT(ch == 16 || ch == 32 || ch == 64, "chunk");
                            EXPECT(st >= LA_OK && st <= LA_ERR_HIP, "plan status");
                        }
    EXPECT(la_forward_plan(1 << 20, 1 << 20, 1 << 20, 128, 128, 1, LA_BF16, 0, NULL, NULL, NULL) != LA_OK,
           "oversized plan refused");
    EXPECT(la_forward_plan(INT64_MAX, 2, 2, 64, 64, 1, LA_F32, 0, NULL, NULL, NULL) != LA_OK, "overflow refused");
    /* forward calls refused by their checks */
    EXPECT(la_forward_chunked(NULL, F, F, F, 1, 1, 64, 16, 16, 1, LA_F32, 0, NULL, 0, NULL, NULL, NULL) ==
               LA_ERR_INVALID_ARG, "null Q");
    EXPECT(la_forward_chunked(F, F, F, F, 1, 1, 64, 40, 16, 1, LA_F32, 0, F, 1 << 20, NULL, NULL, NULL) ==
               LA_ERR_UNSUPPORTED, "width 40");
    EXPECT(la_forward_chunked(F, F, F, F, 1, 1, 4096, 48, 48, 1, LA_F32, 0, NULL, 0, NULL, NULL, NULL) ==
               LA_ERR_WORKSPACE, "padded width without workspace");
    EXPECT(la_forward_chunked(F, F, F, F, 1, 1, 64, 16, 16, 1, LA_F32, 0, NULL, 0, F, NULL, NULL) ==
               LA_ERR_INVALID_ARG, "S_out without z_out");
    EXPECT(la_forward_continue(F, F, F, F, 2, 2, 1000, 64, 64, LA_F32, 0, F, NULL, F, 1 << 30, NULL, NULL, NULL) ==
               LA_ERR_INVALID_ARG, "S_in without z_in");
    EXPECT(la_forward_fused(F, F, F, F, 1, 1, 64, 48, 48, LA_F32, 16, 1, NULL, NULL, NULL, 0, NULL, NULL, NULL) ==
               LA_ERR_UNSUPPORTED, "explicit plan at a padded width");
    EXPECT(la_forward_onepass(F, F, F, F, 1, 1, 1000, 64, 64, LA_F32, 16, 1, NULL, NULL, NULL, 0, NULL, NULL, NULL) ==
               LA_ERR_UNSUPPORTED, "one-pass segment too long");
    EXPECT(la_forward_chunked_noalloc(F, F, F, F, 1, 16, 65536, 112, 112, 1, LA_BF16, 0, NULL, NULL, NULL) ==
               LA_ERR_WORKSPACE, "no-alloc plan beyond the scratch");
    EXPECT(la_noalloc_scratch_bytes() == LA_NOALLOC_SCRATCH_BYTES, "scratch size");
    EXPECT(la_workspace_status(NULL, 64, NULL) == LA_ERR_INVALID_ARG, "status of NULL");
    EXPECT(la_workspace_status(F, 8, NULL) == LA_ERR_INVALID_ARG, "status of a short workspace");
    /* stages, decode, backward, softmax, features, probes */
    EXPECT(la_segment_states(F, F, F, 1 << 20, 1, 1, 64, 16, 16, LA_F32, 16, 0, 0, NULL) == LA_ERR_INVALID_ARG,
           "zero segments");
    EXPECT(la_segment_scan(F, 1 << 20, 1, 1, 48, 16, 2, 2, NULL, NULL, NULL) == LA_ERR_UNSUPPORTED, "scan width");
    EXPECT(la_decode_step(F, F, F, F, F, F, 2, 2, 40, 64, LA_F32, NULL) == LA_ERR_UNSUPPORTED, "decode width 40");
    EXPECT(la_decode_step(F, F, F, F, F, F, 2, 2, 64, 64, 7, NULL) == LA_ERR_INVALID_ARG, "decode dtype");
    EXPECT(la_decode_steps(F, F, F, F, F, F, 2, 2, -1, 64, 64, LA_F32, NULL) == LA_ERR_INVALID_ARG, "negative T");
    EXPECT(la_decode_steps(F, F, F, F, F, F, 2, 2, 0, 48, 48, LA_F32, NULL) == LA_OK, "T = 0");
    EXPECT(la_backward_workspace_bytes(2, 2, 100, 64, 64, LA_F32_FEATURES) ==
               la_backward_workspace_bytes(2, 2, 100, 64, 64, LA_F32), "backward plans features like fp32");
    EXPECT(la_backward_workspace_bytes(2, 2, 100, 64, 64, LA_F32 | LA_OUT_BF16) == 0, "backward refuses bf16 outputs");
    EXPECT(la_feature_map_backward(F, F, F, 100, 64, LA_F32, F, 16, 3, 0, NULL) == LA_ERR_INVALID_ARG,
           "feature map backward kind");
    EXPECT(la_feature_map_backward(F, F, F, 100, 48, LA_F32, F, 16, 1, 0, NULL) == LA_ERR_UNSUPPORTED,
           "feature map backward width");
    EXPECT(la_feature_map_backward(NULL, NULL, NULL, 0, 64, LA_F32, NULL, 16, 1, 0, NULL) == LA_OK,
           "feature map backward no rows");
    EXPECT(la_backward_chunked(F, F, F, F, F, F, F, F, 2, 2, 100, 64, 64, LA_F32, NULL, 0, NULL) == LA_ERR_WORKSPACE,
           "backward workspace");
    EXPECT(la_softmax_scan_workspace_bytes(2, 2, 128, 64, 64) == 0, "one softmax group");
    EXPECT(la_softmax_step(F, F, F, F, F, F, F, 2, 2, 64, 64, LA_F32_FEATURES, NULL) == LA_ERR_INVALID_ARG,
           "softmax dtype");
    EXPECT(la_feature_map(F, F, NULL, NULL, 100, 48, LA_F32, F, 16, LA_FEATURE_PRF, 0, NULL) == LA_ERR_UNSUPPORTED,
           "feature width");
    EXPECT(la_forward_features_workspace_bytes(8, 8, 1024, 48, 64, 16, 1) == 0, "fused feature width");
    EXPECT(la_decode_step_features(F, F, F, F, F, F, 2, 2, 64, 64, LA_F32, F, 24, LA_FEATURE_PRF, 0, NULL) ==
               LA_ERR_UNSUPPORTED, "decode feature count");
    EXPECT(la_probe_copy(NULL, NULL, 20, NULL) == LA_ERR_INVALID_ARG, "copy size");
    EXPECT(la_probe_read(NULL, NULL, 0, NULL) == LA_ERR_INVALID_ARG, "read out");
    EXPECT(la_probe_mfma(NULL, 5, 1, 1, 0.5f, NULL) == LA_ERR_INVALID_ARG, "mfma dtype");
    if (fails) return 1;
    printf("abi sanitizer run ok\n");
    return 0;
}
