/* Host sanitizer run of the fp64 oracle (test infrastructure only): every entry
 * point of oracle.c on small inputs, including the empty and one-position cases,
 * built with AddressSanitizer and UndefinedBehaviorSanitizer.  A memory error or
 * undefined behaviour aborts the run; the few checks below catch a function that
 * leaves its output unwritten (values that must equal a closed form). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_phi(const double *x, double *y, int64_t n);
void oracle_causal(const double *Q, const double *K, const double *V, double *out, double *S_out, double *z_out,
                   int64_t BH, int64_t N, int64_t D, int64_t M, int threads);
void oracle_causal_from(const double *Q, const double *K, const double *V, const double *S0, const double *z0,
                        double *out, double *S_out, double *z_out, int64_t BH, int64_t N, int64_t D, int64_t M,
                        int threads);
void oracle_causal_rows(const double *Q, const double *K, const double *V, int64_t N, int64_t D, int64_t M,
                        const int64_t *rows, int64_t nrows, double *out, int threads);
void oracle_noncausal(const double *Q, const double *K, const double *V, double *out, int64_t BH, int64_t N,
                      int64_t D, int64_t M, int threads);
void oracle_decode_step(double *S, double *z, const double *q, const double *k, const double *v, double *out,
                        int64_t BH, int64_t D, int64_t M, int threads);
void oracle_causal_backward(const double *Q, const double *K, const double *V, const double *dO, double *dQ,
                            double *dK, double *dV, int64_t BH, int64_t N, int64_t D, int64_t M, int threads);
void oracle_softmax_scan(const double *q, const double *K, const double *V, double *out, double *m_out,
                         double *u_out, double *w_out, int64_t BH, int64_t N, int64_t D, int64_t M, int threads);
void oracle_softmax_step(double *m, double *u, double *w, const double *q, const double *k, const double *v,
                         double *out, int64_t BH, int64_t D, int64_t M, int threads);
void oracle_feature_map(const double *X, const double *W, double *out, int64_t rows, int64_t D, int64_t F,
                        int kind, int normalize, int threads);
void oracle_attention_mapped(const double *Fq, const double *Fk, const double *V, double *out, double *S_out,
                             double *z_out, int64_t BH, int64_t N, int64_t F, int64_t M, int causal, int threads);

static uint64_t st = 88172645463325252ull;
static double rnd(void) { /* xorshift64, uniform in [-1, 1) */
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (double)(st >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *arr(int64_t n) { /* exact-size heap blocks so that any overrun is reported */
    double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}
static int fails = 0;
static void expect(int ok, const char *what) {
    if (!ok) { fprintf(stderr, "FAIL %s\n", what); ++fails; }
}

static void run(int64_t BH, int64_t N, int64_t D, int64_t M, int threads) {
    double *Q = arr(BH * N * D), *K = arr(BH * N * D), *V = arr(BH * N * M), *out = arr(BH * N * M);
    double *S = arr(BH * D * M), *z = arr(BH * D), *S0 = arr(BH * D * M), *z0 = arr(BH * D);
    for (int64_t i = 0; i < BH * D; ++i) z0[i] = fabs(z0[i]) + 0.5; /* a valid carried normaliser */
    for (int64_t i = 0; i < BH * D * M; ++i) S0[i] = 0.0;
    oracle_causal(Q, K, V, out, S, z, BH, N, D, M, threads);
    if (N > 0) /* the first row equals v_0 */
        for (int64_t m = 0; m < M; ++m) expect(fabs(out[m] - V[m]) < 1e-12, "causal first row");
    oracle_causal_from(Q, K, V, S0, z0, out, S, z, BH, N, D, M, threads);
    oracle_noncausal(Q, K, V, out, BH, N, D, M, threads);
    if (N > 0) {
        int64_t rows[3] = {0, N / 2, N - 1};
        double *o3 = arr(3 * M);
        oracle_causal_rows(Q, K, V, N, D, M, rows, 3, o3, threads);
        for (int64_t m = 0; m < M; ++m) expect(fabs(o3[m] - V[m]) < 1e-12, "rows first row");
        free(o3);
    }
    double *dO = arr(BH * N * M), *dQ = arr(BH * N * D), *dK = arr(BH * N * D), *dV = arr(BH * N * M);
    oracle_causal_backward(Q, K, V, dO, dQ, dK, dV, BH, N, D, M, threads);
    double *q1 = arr(BH * D), *k1 = arr(BH * D), *v1 = arr(BH * M), *o1 = arr(BH * M);
    for (int64_t i = 0; i < BH * D * M; ++i) S[i] = 0.0;
    for (int64_t i = 0; i < BH * D; ++i) z[i] = 0.0;
    oracle_decode_step(S, z, q1, k1, v1, o1, BH, D, M, threads);
    for (int64_t m = 0; m < M; ++m) expect(fabs(o1[m] - v1[m]) < 1e-12, "decode from zero returns v");
    double *mm = arr(BH), *uu = arr(BH), *ww = arr(BH * M);
    oracle_softmax_scan(q1, K, V, out, mm, uu, ww, BH, N, D, M, threads);
    for (int64_t h = 0; h < BH; ++h) { mm[h] = -INFINITY; uu[h] = 0.0; }
    for (int64_t i = 0; i < BH * M; ++i) ww[i] = 0.0;
    oracle_softmax_step(mm, uu, ww, q1, k1, v1, o1, BH, D, M, threads);
    for (int64_t m = 0; m < M; ++m) expect(fabs(o1[m] - v1[m]) < 1e-12, "softmax step from empty returns v");
    const int64_t F = 16, rows = BH * N;
    double *W = arr(F * D), *Fq = arr(rows * F), *Fk = arr(rows * F), *SF = arr(BH * F * M), *zF = arr(BH * F);
    oracle_feature_map(Q, W, Fq, rows, D, F, 1, 0, threads);
    oracle_feature_map(K, W, Fk, rows, D, F, 2, 1, threads);
    for (int64_t i = 0; i < rows * F; ++i) Fk[i] = fabs(Fk[i]) + 0.1; /* positive features */
    oracle_attention_mapped(Fq, Fk, V, out, SF, zF, BH, N, F, M, 1, threads);
    oracle_attention_mapped(Fk, Fk, V, out, SF, zF, BH, N, F, M, 0, threads);
    double *Xe = arr(rows * D), *Ye = arr(rows * D);
    oracle_feature_map(Q, NULL, Xe, rows, D, D, 0, 0, threads); /* elu + 1 needs no W */
    oracle_phi(Q, Ye, rows * D);
    for (int64_t i = 0; i < rows * D; ++i) expect(Xe[i] == Ye[i], "elu feature map equals phi");
    free(Xe); free(Ye);
    free(Q); free(K); free(V); free(out); free(S); free(z); free(S0); free(z0);
    free(dO); free(dQ); free(dK); free(dV); free(q1); free(k1); free(v1); free(o1);
    free(mm); free(uu); free(ww); free(W); free(Fq); free(Fk); free(SF); free(zF);
}

int main(void) {
    const int64_t shapes[][4] = {{1, 0, 4, 3}, {1, 1, 1, 1}, {2, 1, 3, 5}, {3, 17, 8, 4}, {2, 65, 16, 16}};
    for (int s = 0; s < 5; ++s)
        for (int t = 1; t <= 2; ++t) run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], t);
    if (fails) return 1;
    printf("oracle sanitizer run ok\n");
    return 0;
}
