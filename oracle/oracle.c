/*
 * Oracle for causal kernelized linear attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the bench's CPU-baseline leg may load
 * this library.  The HIP product path never calls it and shares no code with it.
 *
 * Everything is float64 on the host, written as plainly as possible so that it
 * can be checked against the pages by eye.  The method is that of
 * "Transformers are RNNs: Fast Autoregressive Transformers with Linear Attention"
 * (Katharopoulos et al., 2020), as reviewed on the page of that title:
 *
 *   - Proposed method: softmax similarity is replaced by a dot product of feature
 *     maps phi(q)^T phi(k); by associativity the attention becomes
 *     phi(Q) (phi(K)^T V), a sum computed once and reused by every query.
 *   - Proposed method: causal masking is kept by updating the cumulative sums
 *     S_i and Z_i one position at a time (linear time, constant memory); the
 *     causal model is an RNN with the two memories (S, z).
 *   - Main findings: the feature map is elu based; phi(x) = elu(x) + 1.
 *
 * With S_i = sum_{j<=i} phi(k_j) v_j^T (D x M) and z_i = sum_{j<=i} phi(k_j) (D):
 *     out_i = phi(q_i)^T S_i / (phi(q_i)^T z_i).
 *
 * Layouts (row major, contiguous): Q, K [BH][N][D]; V, out [BH][N][M];
 * S [BH][D][M] (row d, column m); z [BH][D].
 *
 * Every function here is pinned by tests outside this file (hand-derived exact
 * values, closed forms, invariants and 50-digit evaluations); none is "parity
 * unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* phi(x) = elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise.
 * (Page "Transformers are RNNs", Main findings: elu-based feature map.)
 * The exp branch is elu(x) + 1 = (exp(x) - 1) + 1 written without the
 * cancellation. */
double oracle_phi1(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

void oracle_phi(const double *x, double *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_phi1(x[i]);
}

static int pick_threads(int threads) {
#ifdef _OPENMP
    return threads > 0 ? threads : omp_get_max_threads();
#else
    (void)threads;
    return 1;
#endif
}

int oracle_max_threads(void) { return pick_threads(0); }

/* Causal attention by the running sums of the page (Proposed method: S_i and
 * Z_i updated step by step).  Per head: S = 0, z = 0; for i = 0..N-1 add
 * phi(k_i) v_i^T to S and phi(k_i) to z, then read out with phi(q_i).
 * S_out / z_out (may be NULL) receive the final state S_{N-1}, z_{N-1}. */
void oracle_causal(const double *Q, const double *K, const double *V, double *out,
                   double *S_out, double *z_out,
                   int64_t BH, int64_t N, int64_t D, int64_t M, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        double *S = (double *)calloc((size_t)(D * M), sizeof(double));
        double *z = (double *)calloc((size_t)D, sizeof(double));
        double *f = (double *)malloc((size_t)D * sizeof(double));
        double *g = (double *)malloc((size_t)D * sizeof(double));
        const double *Qh = Q + h * N * D, *Kh = K + h * N * D, *Vh = V + h * N * M;
        double *Oh = out + h * N * M;
        for (int64_t i = 0; i < N; ++i) {
            const double *k = Kh + i * D, *q = Qh + i * D, *v = Vh + i * M;
            for (int64_t d = 0; d < D; ++d) f[d] = oracle_phi1(k[d]);
            for (int64_t d = 0; d < D; ++d) {
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += f[d] * v[m];
                z[d] += f[d];
            }
            for (int64_t d = 0; d < D; ++d) g[d] = oracle_phi1(q[d]);
            double den = 0.0;
            for (int64_t d = 0; d < D; ++d) den += g[d] * z[d];
            for (int64_t m = 0; m < M; ++m) {
                double num = 0.0;
                for (int64_t d = 0; d < D; ++d) num += g[d] * S[d * M + m];
                Oh[i * M + m] = num / den;
            }
        }
        if (S_out) memcpy(S_out + h * D * M, S, (size_t)(D * M) * sizeof(double));
        if (z_out) memcpy(z_out + h * D, z, (size_t)D * sizeof(double));
        free(S); free(z); free(f); free(g);
    }
}

/* Causal attention continued from a carried state: the same running sums, but
 * the memories start at (S0, z0) -- the state left by the positions before this
 * block -- instead of zero.  (Page "Transformers are RNNs", Proposed method: the
 * causal model is an RNN whose memories S and z carry all earlier positions.)
 * S0 [BH][D][M], z0 [BH][D]; S_out / z_out (may be NULL) receive the final state. */
void oracle_causal_from(const double *Q, const double *K, const double *V,
                        const double *S0, const double *z0, double *out,
                        double *S_out, double *z_out,
                        int64_t BH, int64_t N, int64_t D, int64_t M, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        double *S = (double *)malloc((size_t)(D * M) * sizeof(double));
        double *z = (double *)malloc((size_t)D * sizeof(double));
        memcpy(S, S0 + h * D * M, (size_t)(D * M) * sizeof(double));
        memcpy(z, z0 + h * D, (size_t)D * sizeof(double));
        const double *Qh = Q + h * N * D, *Kh = K + h * N * D, *Vh = V + h * N * M;
        double *Oh = out + h * N * M;
        for (int64_t i = 0; i < N; ++i) {
            const double *k = Kh + i * D, *q = Qh + i * D, *v = Vh + i * M;
            for (int64_t d = 0; d < D; ++d) {
                double f = oracle_phi1(k[d]);
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += f * v[m];
                z[d] += f;
            }
            double den = 0.0;
            for (int64_t d = 0; d < D; ++d) den += oracle_phi1(q[d]) * z[d];
            for (int64_t m = 0; m < M; ++m) {
                double num = 0.0;
                for (int64_t d = 0; d < D; ++d) num += oracle_phi1(q[d]) * S[d * M + m];
                Oh[i * M + m] = num / den;
            }
        }
        if (S_out) memcpy(S_out + h * D * M, S, (size_t)(D * M) * sizeof(double));
        if (z_out) memcpy(z_out + h * D, z, (size_t)D * sizeof(double));
        free(S); free(z);
    }
}

/* Causal attention straight from its definition, for selected rows of ONE head:
 *   out_i = sum_{j<=i} (phi(q_i).phi(k_j)) v_j / sum_{j<=i} phi(q_i).phi(k_j).
 * (Page "Transformers are RNNs", Proposed method: the softmax similarity is
 * replaced by the feature-map dot product; causal masking keeps j <= i.)
 * Cost O(i (D + M)) per row, so single rows of very long sequences can be
 * checked one by one.  Q, K: [N][D], V: [N][M], out: [nrows][M]. */
void oracle_causal_rows(const double *Q, const double *K, const double *V,
                        int64_t N, int64_t D, int64_t M,
                        const int64_t *rows, int64_t nrows, double *out, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows[r];
        double *o = out + r * M;
        if (i < 0 || i >= N) {
            for (int64_t m = 0; m < M; ++m) o[m] = NAN;
            continue;
        }
        double *g = (double *)malloc((size_t)D * sizeof(double));
        double *num = (double *)calloc((size_t)M, sizeof(double));
        for (int64_t d = 0; d < D; ++d) g[d] = oracle_phi1(Q[i * D + d]);
        double den = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
            double w = 0.0;
            for (int64_t d = 0; d < D; ++d) w += g[d] * oracle_phi1(K[j * D + d]);
            for (int64_t m = 0; m < M; ++m) num[m] += w * V[j * M + m];
            den += w;
        }
        for (int64_t m = 0; m < M; ++m) o[m] = num[m] / den;
        free(g); free(num);
    }
}

/* Non-causal attention in the associative form of the page (Proposed method:
 * phi(Q) (phi(K)^T V), the sum computed once and reused for every query):
 * S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j); out_i = phi(q_i)^T S / phi(q_i).z. */
void oracle_noncausal(const double *Q, const double *K, const double *V, double *out,
                      int64_t BH, int64_t N, int64_t D, int64_t M, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        double *S = (double *)calloc((size_t)(D * M), sizeof(double));
        double *z = (double *)calloc((size_t)D, sizeof(double));
        double *g = (double *)malloc((size_t)D * sizeof(double));
        const double *Qh = Q + h * N * D, *Kh = K + h * N * D, *Vh = V + h * N * M;
        double *Oh = out + h * N * M;
        for (int64_t j = 0; j < N; ++j) {
            for (int64_t d = 0; d < D; ++d) {
                double f = oracle_phi1(Kh[j * D + d]);
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += f * Vh[j * M + m];
                z[d] += f;
            }
        }
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t d = 0; d < D; ++d) g[d] = oracle_phi1(Qh[i * D + d]);
            double den = 0.0;
            for (int64_t d = 0; d < D; ++d) den += g[d] * z[d];
            for (int64_t m = 0; m < M; ++m) {
                double num = 0.0;
                for (int64_t d = 0; d < D; ++d) num += g[d] * S[d * M + m];
                Oh[i * M + m] = num / den;
            }
        }
        free(S); free(z); free(g);
    }
}

/* One recurrent (autoregressive) step for BH independent heads.
 * (Page "Transformers are RNNs", Proposed method: the causal transformer is an
 * RNN with the memories (S, z); Main findings: the internal state is updated
 * incrementally.)  The new token enters the state first, then the output is read
 * (the sums run over j <= i): S += phi(k) v^T; z += phi(k);
 * out = phi(q)^T S / phi(q).z.  S [BH][D][M] and z [BH][D] are updated in place;
 * q, k [BH][D]; v, out [BH][M]. */
void oracle_decode_step(double *S, double *z, const double *q, const double *k,
                        const double *v, double *out,
                        int64_t BH, int64_t D, int64_t M, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        double *Sh = S + h * D * M, *zh = z + h * D;
        const double *qh = q + h * D, *kh = k + h * D, *vh = v + h * M;
        double *oh = out + h * M;
        for (int64_t d = 0; d < D; ++d) {
            double f = oracle_phi1(kh[d]);
            for (int64_t m = 0; m < M; ++m) Sh[d * M + m] += f * vh[m];
            zh[d] += f;
        }
        double den = 0.0;
        for (int64_t d = 0; d < D; ++d) den += oracle_phi1(qh[d]) * zh[d];
        for (int64_t m = 0; m < M; ++m) {
            double num = 0.0;
            for (int64_t d = 0; d < D; ++d) num += oracle_phi1(qh[d]) * Sh[d * M + m];
            oh[m] = num / den;
        }
    }
}

/* Derivative of phi: 1 for x > 0, exp(x) otherwise (continuous, 1 at 0). */
static double oracle_dphi1(double x) { return x > 0.0 ? 1.0 : exp(x); }

/* Gradients of causal attention (the training half of the parallel mode; page
 * "Transformers are RNNs", Proposed method: gradients in linear time, so that
 * training keeps constant memory like the forward running sums).
 * The chain rule through out_i = num_i / den_i with num_i = phi(q_i)^T S_i and
 * den_i = phi(q_i)^T z_i gives, with g_i = phi(q_i), f_j = phi(k_j),
 *   r_i = dout_i / den_i  (M),  c_i = -(dout_i . out_i) / den_i,
 *   dL/dg_i = S_i r_i + c_i z_i                          (sums over j <= i)
 *   dL/df_j = R_j v_j + w_j,  dL/dv_j = R_j^T f_j        (sums over i >= j)
 * where R_j = sum_{i>=j} g_i r_i^T (D x M) and w_j = sum_{i>=j} c_i g_i (D):
 * a forward running sum for the query side and a reverse one for the key and
 * value side.  Then dq = dL/dg * phi'(q), dk = dL/df * phi'(k).
 * dO [BH][N][M] (the output gradient); dQ, dK [BH][N][D], dV [BH][N][M]. */
void oracle_causal_backward(const double *Q, const double *K, const double *V, const double *dO,
                            double *dQ, double *dK, double *dV,
                            int64_t BH, int64_t N, int64_t D, int64_t M, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const double *Qh = Q + h * N * D, *Kh = K + h * N * D, *Vh = V + h * N * M, *dOh = dO + h * N * M;
        double *dQh = dQ + h * N * D, *dKh = dK + h * N * D, *dVh = dV + h * N * M;
        double *S = (double *)calloc((size_t)(D * M), sizeof(double));
        double *z = (double *)calloc((size_t)D, sizeof(double));
        double *r = (double *)malloc((size_t)(N * M) * sizeof(double));
        double *c = (double *)malloc((size_t)N * sizeof(double));
        double *o = (double *)malloc((size_t)M * sizeof(double));
        /* forward running sums: outputs, r_i, c_i and the query-side gradient */
        for (int64_t i = 0; i < N; ++i) {
            const double *q = Qh + i * D, *k = Kh + i * D, *v = Vh + i * M, *dout = dOh + i * M;
            for (int64_t d = 0; d < D; ++d) {
                double f = oracle_phi1(k[d]);
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += f * v[m];
                z[d] += f;
            }
            double den = 0.0;
            for (int64_t d = 0; d < D; ++d) den += oracle_phi1(q[d]) * z[d];
            double dot = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                double num = 0.0;
                for (int64_t d = 0; d < D; ++d) num += oracle_phi1(q[d]) * S[d * M + m];
                o[m] = num / den;
                dot += dout[m] * o[m];
            }
            for (int64_t m = 0; m < M; ++m) r[i * M + m] = dout[m] / den;
            c[i] = -dot / den;
            for (int64_t d = 0; d < D; ++d) {
                double dg = c[i] * z[d];
                for (int64_t m = 0; m < M; ++m) dg += S[d * M + m] * r[i * M + m];
                dQh[i * D + d] = dg * oracle_dphi1(q[d]);
            }
        }
        /* reverse running sums: key- and value-side gradients */
        double *R = S, *w = z; /* reused, cleared */
        memset(R, 0, (size_t)(D * M) * sizeof(double));
        memset(w, 0, (size_t)D * sizeof(double));
        for (int64_t j = N - 1; j >= 0; --j) {
            const double *q = Qh + j * D, *k = Kh + j * D, *v = Vh + j * M;
            for (int64_t d = 0; d < D; ++d) {
                double g = oracle_phi1(q[d]);
                for (int64_t m = 0; m < M; ++m) R[d * M + m] += g * r[j * M + m];
                w[d] += c[j] * g;
            }
            for (int64_t d = 0; d < D; ++d) {
                double df = w[d];
                for (int64_t m = 0; m < M; ++m) df += R[d * M + m] * v[m];
                dKh[j * D + d] = df * oracle_dphi1(k[d]);
            }
            for (int64_t m = 0; m < M; ++m) {
                double dv = 0.0;
                for (int64_t d = 0; d < D; ++d) dv += R[d * M + m] * oracle_phi1(k[d]);
                dVh[j * M + m] = dv;
            }
        }
        free(S); free(z); free(r); free(c); free(o);
    }
}

/* Softmax attention of one query per head over every prefix, as an RNN
 * (page "Attention as an RNN", Proposed method: attention is an RNN whose
 * many-to-many outputs -- the attention of the query over each prefix -- are
 * computed with a running state; the query is a learned vector q).  With
 * s_i = q . k_i (no scaling; a caller scales q), the state after position k is
 * (m_k, u_k, w_k) = (max_{i<=k} s_i, sum_{i<=k} exp(s_i - m_k),
 * sum_{i<=k} exp(s_i - m_k) v_i), updated position by position:
 *   m' = max(m, s);  u' = u e^{m - m'} + e^{s - m'};  w' = w e^{m - m'} + e^{s - m'} v
 * and out_k = w_k / u_k.  q [BH][D]; K [BH][N][D]; V, out [BH][N][M];
 * m_out, u_out [BH], w_out [BH][M] (may be NULL): the final state. */
void oracle_softmax_scan(const double *q, const double *K, const double *V, double *out,
                         double *m_out, double *u_out, double *w_out,
                         int64_t BH, int64_t N, int64_t D, int64_t M, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const double *qh = q + h * D, *Kh = K + h * N * D, *Vh = V + h * N * M;
        double *Oh = out + h * N * M;
        double *w = (double *)calloc((size_t)M, sizeof(double));
        double m = -INFINITY, u = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            double s = 0.0;
            for (int64_t d = 0; d < D; ++d) s += qh[d] * Kh[i * D + d];
            const double mn = m > s ? m : s;
            const double a = exp(m - mn), b = exp(s - mn);
            u = u * a + b;
            for (int64_t j = 0; j < M; ++j) {
                w[j] = w[j] * a + b * Vh[i * M + j];
                Oh[i * M + j] = w[j] / u;
            }
            m = mn;
        }
        if (m_out) m_out[h] = m;
        if (u_out) u_out[h] = u;
        if (w_out) memcpy(w_out + h * M, w, (size_t)M * sizeof(double));
        free(w);
    }
}

/* One token of the same RNN for BH heads (constant memory): the state
 * (m [BH], u [BH], w [BH][M]) is updated in place with (k, v) and the output is
 * the attention of q over every token seen so far.  q, k [BH][D]; v, out [BH][M].
 * A fresh state is m = -inf, u = 0, w = 0. */
void oracle_softmax_step(double *m, double *u, double *w, const double *q, const double *k,
                         const double *v, double *out, int64_t BH, int64_t D, int64_t M, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        double s = 0.0;
        for (int64_t d = 0; d < D; ++d) s += q[h * D + d] * k[h * D + d];
        const double mn = m[h] > s ? m[h] : s;
        const double a = exp(m[h] - mn), b = exp(s - mn);
        u[h] = u[h] * a + b;
        for (int64_t j = 0; j < M; ++j) {
            w[h * M + j] = w[h * M + j] * a + b * v[h * M + j];
            out[h * M + j] = w[h * M + j] / u[h];
        }
        m[h] = mn;
    }
}

/* Random-feature maps with feature dimension F (page "Stable, Fast and Accurate:
 * Kernelized Attention with Relative Positional Encoding", Proposed method and
 * Main findings: kernelized attention with the feature maps PRF, TRF,
 * Sphere-PRF and ORF, feature dimension as small as 16; normalised queries and
 * keys for large norms).  The page gives no formula; these are the published
 * random-feature estimators of the softmax kernel exp(q . k), whose expected
 * dot product phi(q) . phi(k) over w ~ N(0, I) is exactly exp(q . k):
 *   kind 0 (elu):  phi(x) = elu(x) + 1 elementwise, F = D, W unused;
 *   kind 1 (PRF, positive):      phi_f(x) = exp(w_f . x - |x|^2 / 2) / sqrt(F),
 *                                W [F][D];
 *   kind 2 (TRF, trigonometric): with P = F / 2 projections W [P][D] and
 *                                c(x) = exp(|x|^2 / 2) / sqrt(P):
 *                                phi_p(x) = c sin(w_p . x), phi_{P+p}(x) = c cos(w_p . x).
 * ORF and Sphere-PRF are PRF with a differently drawn W (orthogonal rows; rows on
 * a sphere), which the caller passes in.  normalize != 0 first scales every row
 * x to unit length (x = 0 stays 0).  X [rows][D]; out [rows][F]. */
void oracle_feature_map(const double *X, const double *W, double *out, int64_t rows, int64_t D, int64_t F,
                        int kind, int normalize, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r) {
        double *x = (double *)malloc((size_t)D * sizeof(double));
        double sq = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            x[d] = X[r * D + d];
            sq += x[d] * x[d];
        }
        if (normalize && sq > 0.0) {
            const double len = sqrt(sq);
            sq = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                x[d] /= len;
                sq += x[d] * x[d];
            }
        }
        double *o = out + r * F;
        if (kind == 0) {
            for (int64_t d = 0; d < D; ++d) o[d] = oracle_phi1(x[d]);
        } else if (kind == 1) {
            for (int64_t f = 0; f < F; ++f) {
                double p = 0.0;
                for (int64_t d = 0; d < D; ++d) p += W[f * D + d] * x[d];
                o[f] = exp(p - 0.5 * sq) / sqrt((double)F);
            }
        } else {
            const int64_t P = F / 2;
            const double c = exp(0.5 * sq) / sqrt((double)P);
            for (int64_t p = 0; p < P; ++p) {
                double a = 0.0;
                for (int64_t d = 0; d < D; ++d) a += W[p * D + d] * x[d];
                o[p] = c * sin(a);
                o[P + p] = c * cos(a);
            }
        }
        free(x);
    }
}

/* Linear attention on features that are already mapped (Fq = phi(Q), Fk = phi(K),
 * [BH][N][F]): the running sums of the page "Transformers are RNNs" (Proposed
 * method) with no feature map applied.  causal != 0: S_i, z_i over j <= i, read
 * out with Fq_i after position i enters; causal == 0: the sums over all j, read
 * out once per row.  S_out [BH][F][M], z_out [BH][F] (may be NULL): the sums over
 * all N positions. */
void oracle_attention_mapped(const double *Fq, const double *Fk, const double *V, double *out, double *S_out,
                             double *z_out, int64_t BH, int64_t N, int64_t F, int64_t M, int causal,
                             int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        double *S = (double *)calloc((size_t)(F * M), sizeof(double));
        double *z = (double *)calloc((size_t)F, sizeof(double));
        const double *Qh = Fq + h * N * F, *Kh = Fk + h * N * F, *Vh = V + h * N * M;
        double *Oh = out + h * N * M;
        if (causal) {
            /* add position i, then read out row i */
            for (int64_t i = 0; i < N; ++i) {
                const double *f = Kh + i * F, *g = Qh + i * F, *v = Vh + i * M;
                for (int64_t d = 0; d < F; ++d) {
                    for (int64_t m = 0; m < M; ++m) S[d * M + m] += f[d] * v[m];
                    z[d] += f[d];
                }
                double den = 0.0;
                for (int64_t d = 0; d < F; ++d) den += g[d] * z[d];
                for (int64_t m = 0; m < M; ++m) {
                    double num = 0.0;
                    for (int64_t d = 0; d < F; ++d) num += g[d] * S[d * M + m];
                    Oh[i * M + m] = num / den;
                }
            }
        } else {
            /* add every position, then read out every row */
            for (int64_t j = 0; j < N; ++j) {
                const double *f = Kh + j * F, *v = Vh + j * M;
                for (int64_t d = 0; d < F; ++d) {
                    for (int64_t m = 0; m < M; ++m) S[d * M + m] += f[d] * v[m];
                    z[d] += f[d];
                }
            }
            for (int64_t i = 0; i < N; ++i) {
                const double *g = Qh + i * F;
                double den = 0.0;
                for (int64_t d = 0; d < F; ++d) den += g[d] * z[d];
                for (int64_t m = 0; m < M; ++m) {
                    double num = 0.0;
                    for (int64_t d = 0; d < F; ++d) num += g[d] * S[d * M + m];
                    Oh[i * M + m] = num / den;
                }
            }
        }
        if (S_out) memcpy(S_out + h * F * M, S, (size_t)(F * M) * sizeof(double));
        if (z_out) memcpy(z_out + h * F, z, (size_t)F * sizeof(double));
        free(S); free(z);
    }
}

/* Gradients of causal linear attention on mapped features (Fq = phi(Q), Fk = phi(K)
 * already formed, [BH][N][F]; no feature map inside): the running-sum gradients of
 * oracle_causal_backward with phi the identity, so phi' = 1 and the results are the
 * gradients with respect to the features themselves (page "Transformers are RNNs",
 * Proposed method: gradients by running sums in linear time).  dFq, dFk [BH][N][F],
 * dV [BH][N][M]. */
void oracle_backward_mapped(const double *Fq, const double *Fk, const double *V, const double *dO,
                            double *dFq, double *dFk, double *dV,
                            int64_t BH, int64_t N, int64_t F, int64_t M, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t h = 0; h < BH; ++h) {
        const double *Gh = Fq + h * N * F, *Fh = Fk + h * N * F, *Vh = V + h * N * M, *dOh = dO + h * N * M;
        double *dGh = dFq + h * N * F, *dFh = dFk + h * N * F, *dVh = dV + h * N * M;
        double *S = (double *)calloc((size_t)(F * M), sizeof(double));
        double *z = (double *)calloc((size_t)F, sizeof(double));
        double *r = (double *)malloc((size_t)(N * M) * sizeof(double));
        double *c = (double *)malloc((size_t)N * sizeof(double));
        /* forward running sums: r_i = dout_i / den_i, c_i = -(dout_i . out_i) / den_i,
         * and dL/dg_i = S_i r_i + c_i z_i */
        for (int64_t i = 0; i < N; ++i) {
            const double *g = Gh + i * F, *f = Fh + i * F, *v = Vh + i * M, *dout = dOh + i * M;
            for (int64_t d = 0; d < F; ++d) {
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += f[d] * v[m];
                z[d] += f[d];
            }
            double den = 0.0;
            for (int64_t d = 0; d < F; ++d) den += g[d] * z[d];
            double dot = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                double num = 0.0;
                for (int64_t d = 0; d < F; ++d) num += g[d] * S[d * M + m];
                dot += dout[m] * (num / den);
            }
            for (int64_t m = 0; m < M; ++m) r[i * M + m] = dout[m] / den;
            c[i] = -dot / den;
            for (int64_t d = 0; d < F; ++d) {
                double dg = c[i] * z[d];
                for (int64_t m = 0; m < M; ++m) dg += S[d * M + m] * r[i * M + m];
                dGh[i * F + d] = dg;
            }
        }
        /* reverse running sums R_j = sum_{i>=j} g_i r_i^T, w_j = sum_{i>=j} c_i g_i:
         * dL/df_j = R_j v_j + w_j, dL/dv_j = R_j^T f_j */
        memset(S, 0, (size_t)(F * M) * sizeof(double));
        memset(z, 0, (size_t)F * sizeof(double));
        for (int64_t j = N - 1; j >= 0; --j) {
            const double *g = Gh + j * F, *f = Fh + j * F, *v = Vh + j * M;
            for (int64_t d = 0; d < F; ++d) {
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += g[d] * r[j * M + m];
                z[d] += c[j] * g[d];
            }
            for (int64_t d = 0; d < F; ++d) {
                double df = z[d];
                for (int64_t m = 0; m < M; ++m) df += S[d * M + m] * v[m];
                dFh[j * F + d] = df;
            }
            for (int64_t m = 0; m < M; ++m) {
                double dv = 0.0;
                for (int64_t d = 0; d < F; ++d) dv += S[d * M + m] * f[d];
                dVh[j * M + m] = dv;
            }
        }
        free(S); free(z); free(r); free(c);
    }
}

/* Gradient of the feature map of oracle_feature_map with respect to its input rows:
 * dX = J(x)^T dOut row by row, by the chain rule through the definitions there
 * (page "Stable, Fast and Accurate: Kernelized Attention with Relative Positional
 * Encoding", Proposed method: the PRF and TRF maps).  With y the (normalised) row:
 *   elu:  d out_d / d y_d = 1 for y_d > 0, exp(y_d) otherwise;
 *   PRF:  out_f = exp(w_f . y - |y|^2 / 2) / sqrt(F), so
 *         d out_f / d y = out_f (w_f - y);
 *   TRF:  out_p = c sin(a_p), out_{P+p} = c cos(a_p), a_p = w_p . y,
 *         c = exp(|y|^2 / 2) / sqrt(P), d c / d y = c y, so
 *         d out_p / d y = y out_p + c cos(a_p) w_p,
 *         d out_{P+p} / d y = y out_{P+p} - c sin(a_p) w_p.
 * normalize != 0: y = x / |x|, and d y / d x = (I - y y^T) / |x|; a zero row
 * (where the normalisation is not differentiable) gets a zero gradient.
 * X [rows][D]; dOut [rows][F]; dX [rows][D]. */
void oracle_feature_map_backward(const double *X, const double *W, const double *dOut, double *dX, int64_t rows,
                                 int64_t D, int64_t F, int kind, int normalize, int threads) {
    int nt = pick_threads(threads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r) {
        double *y = (double *)malloc((size_t)D * sizeof(double));
        double *dy = (double *)calloc((size_t)D, sizeof(double));
        double sq = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            y[d] = X[r * D + d];
            sq += y[d] * y[d];
        }
        const double len = sqrt(sq);
        const int scaled = normalize && sq > 0.0;
        if (scaled) {
            sq = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                y[d] /= len;
                sq += y[d] * y[d];
            }
        }
        const double *g = dOut + r * F;
        if (kind == 0) {
            for (int64_t d = 0; d < D; ++d) dy[d] = g[d] * (y[d] > 0.0 ? 1.0 : exp(y[d]));
        } else if (kind == 1) {
            for (int64_t f = 0; f < F; ++f) {
                double a = 0.0;
                for (int64_t d = 0; d < D; ++d) a += W[f * D + d] * y[d];
                const double out_f = exp(a - 0.5 * sq) / sqrt((double)F);
                for (int64_t d = 0; d < D; ++d) dy[d] += g[f] * out_f * (W[f * D + d] - y[d]);
            }
        } else {
            const int64_t P = F / 2;
            const double c = exp(0.5 * sq) / sqrt((double)P);
            for (int64_t p = 0; p < P; ++p) {
                double a = 0.0;
                for (int64_t d = 0; d < D; ++d) a += W[p * D + d] * y[d];
                const double s = sin(a), co = cos(a);
                for (int64_t d = 0; d < D; ++d) {
                    dy[d] += g[p] * (y[d] * c * s + c * co * W[p * D + d]);
                    dy[d] += g[P + p] * (y[d] * c * co - c * s * W[p * D + d]);
                }
            }
        }
        double *dx = dX + r * D;
        if (normalize) {
            if (scaled) {
                double ydy = 0.0;
                for (int64_t d = 0; d < D; ++d) ydy += y[d] * dy[d];
                for (int64_t d = 0; d < D; ++d) dx[d] = (dy[d] - y[d] * ydy) / len;
            } else {
                for (int64_t d = 0; d < D; ++d) dx[d] = 0.0;
            }
        } else {
            for (int64_t d = 0; d < D; ++d) dx[d] = dy[d];
        }
        free(y);
        free(dy);
    }
}
