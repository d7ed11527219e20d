"""The oracle against its pins, and the pins against planted mistakes (CPU only)."""
import os

import numpy as np
import pytest

import oracle
import oracle_pins

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    fails = oracle_pins.run_all(oracle.default(), pins=[pin])
    assert not fails, "\n".join(fails)


# Plausible mistakes, each planted in a copy of oracle.c; the pins must catch every one.
MUTANTS = {
    "elu_without_plus_one": ("return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x : exp(x) - 1.0;"),
    "exp_feature_map": ("return x > 0.0 ? x + 1.0 : exp(x);", "return exp(x);"),
    "phi_branch_sign": ("return x > 0.0 ? x + 1.0 : exp(x);", "return x < 0.0 ? x + 1.0 : exp(x);"),
    "dropped_normaliser": ("Oh[i * M + m] = num / den;\n            }\n        }\n        if (S_out)",
                           "Oh[i * M + m] = num;\n            }\n        }\n        if (S_out)"),
    "transposed_state_update": ("for (int64_t m = 0; m < M; ++m) S[d * M + m] += f[d] * v[m];",
                                "for (int64_t m = 0; m < M; ++m) S[m * D + d] += f[d] * v[m];"),
    "numerator_sign": ("for (int64_t d = 0; d < D; ++d) num += g[d] * S[d * M + m];\n                Oh[i * M + m]",
                       "for (int64_t d = 0; d < D; ++d) num -= g[d] * S[d * M + m];\n                Oh[i * M + m]"),
    "exclusive_mask_rows": ("for (int64_t j = 0; j <= i; ++j) {", "for (int64_t j = 0; j < i; ++j) {"),
    "query_key_swap_rows": ("w += g[d] * oracle_phi1(K[j * D + d]);", "w += g[d] * oracle_phi1(Q[j * D + d]);"),
    "value_index_rows": ("num[m] += w * V[j * M + m];", "num[m] += w * V[i * M + m];"),
    "noncausal_wrong_z": ("for (int64_t d = 0; d < D; ++d) den += g[d] * z[d];\n            for (int64_t m = 0; m < M; ++m) {\n                double num = 0.0;\n                for (int64_t d = 0; d < D; ++d) num += g[d] * S[d * M + m];\n                Oh[i * M + m] = num / den;\n            }\n        }\n        free(S); free(z); free(g);",
                          "for (int64_t d = 0; d < D; ++d) den += g[d] * z[0];\n            for (int64_t m = 0; m < M; ++m) {\n                double num = 0.0;\n                for (int64_t d = 0; d < D; ++d) num += g[d] * S[d * M + m];\n                Oh[i * M + m] = num / den;\n            }\n        }\n        free(S); free(z); free(g);"),
    "decode_overwrites_z": ("zh[d] += f;", "zh[d] = f;"),
    "backward_c_sign": ("c[i] = -dot / den;", "c[i] = dot / den;"),
    "backward_dq_phi_not_derivative": ("dQh[i * D + d] = dg * oracle_dphi1(q[d]);",
                                       "dQh[i * D + d] = dg * oracle_phi1(q[d]);"),
    "backward_dv_uses_q": ("dv += R[d * M + m] * oracle_phi1(k[d]);", "dv += R[d * M + m] * oracle_phi1(q[d]);"),
    "backward_missing_w": ("double df = w[d];", "double df = 0.0;"),
    "backward_dk_no_chain_rule": ("dKh[j * D + d] = df * oracle_dphi1(k[d]);", "dKh[j * D + d] = df;"),
    "backward_reverse_sum_exclusive": (
        "                for (int64_t m = 0; m < M; ++m) R[d * M + m] += g * r[j * M + m];\n                w[d] += c[j] * g;\n            }\n            for (int64_t d = 0; d < D; ++d) {\n                double df = w[d];",
        "                for (int64_t m = 0; m < M; ++m) R[d * M + m] += 0.0 * g * r[j * M + m];\n                w[d] += c[j] * g;\n            }\n            for (int64_t d = 0; d < D; ++d) {\n                double df = w[d];"),
    "softmax_w_not_rescaled": ("                w[j] = w[j] * a + b * Vh[i * M + j];", "                w[j] = w[j] + b * Vh[i * M + j];"),
    "softmax_max_not_carried": ("                Oh[i * M + j] = w[j] / u;\n            }\n            m = mn;", "                Oh[i * M + j] = w[j] / u;\n            }\n            m = 0.0;"),
    "softmax_rescale_sign": ("            const double a = exp(m - mn), b = exp(s - mn);\n            u = u * a + b;", "            const double a = exp(mn - m), b = exp(s - mn);\n            u = u * a + b;"),
    "softmax_step_u_not_rescaled": ("        u[h] = u[h] * a + b;", "        u[h] = u[h] + b;"),
    "continue_ignores_z0": ("memcpy(z, z0 + h * D, (size_t)D * sizeof(double));",
                            "memset(z, 0, (size_t)D * sizeof(double));"),
    "continue_ignores_S0": ("memcpy(S, S0 + h * D * M, (size_t)(D * M) * sizeof(double));",
                            "memset(S, 0, (size_t)(D * M) * sizeof(double));"),
    "continue_transposed_update": ("for (int64_t m = 0; m < M; ++m) S[d * M + m] += f * v[m];",
                                   "for (int64_t m = 0; m < M; ++m) S[m * D + d] += f * v[m];"),
    "prf_norm_sign": ("o[f] = exp(p - 0.5 * sq) / sqrt((double)F);", "o[f] = exp(p + 0.5 * sq) / sqrt((double)F);"),
    "prf_no_scale": ("o[f] = exp(p - 0.5 * sq) / sqrt((double)F);", "o[f] = exp(p - 0.5 * sq);"),
    "trf_cos_as_sin": ("o[P + p] = c * cos(a);", "o[P + p] = c * sin(a);"),
    "trf_no_magnitude": ("const double c = exp(0.5 * sq) / sqrt((double)P);", "const double c = 1.0 / sqrt((double)P);"),
    "normalize_ignored": ("if (normalize && sq > 0.0) {", "if (0 && normalize && sq > 0.0) {"),
    "normalize_keeps_old_norm": ("            sq = 0.0;\n            for (int64_t d = 0; d < D; ++d) {\n                x[d] /= len;",
                                 "            for (int64_t d = 0; d < D; ++d) {\n                x[d] /= len;"),
    "mapped_causal_as_noncausal": ("        if (causal) {\n            /* add position i, then read out row i */",
                                   "        if (0) {\n            /* add position i, then read out row i */"),
    "mapped_den_uses_k": ("for (int64_t d = 0; d < F; ++d) den += g[d] * z[d];",
                          "for (int64_t d = 0; d < F; ++d) den += f[d] * z[d];"),
    "mapped_noncausal_sums_q": ("const double *f = Kh + j * F, *v = Vh + j * M;",
                                "const double *f = Qh + j * F, *v = Vh + j * M;"),
    "mapped_backward_c_sign": ("c[i] = -dot / den;\n            for (int64_t d = 0; d < F; ++d) {",
                               "c[i] = dot / den;\n            for (int64_t d = 0; d < F; ++d) {"),
    "mapped_backward_dq_missing_z": ("double dg = c[i] * z[d];\n                for (int64_t m = 0; m < M; ++m) dg += S[d * M + m] * r[i * M + m];\n                dGh",
                                     "double dg = 0.0;\n                for (int64_t m = 0; m < M; ++m) dg += S[d * M + m] * r[i * M + m];\n                dGh"),
    "mapped_backward_missing_w": ("double df = z[d];", "double df = 0.0;"),
    "mapped_backward_dv_uses_g": ("dv += S[d * M + m] * f[d];", "dv += S[d * M + m] * g[d];"),
    "fmb_prf_drops_minus_y": ("dy[d] += g[f] * out_f * (W[f * D + d] - y[d]);", "dy[d] += g[f] * out_f * W[f * D + d];"),
    "fmb_prf_scale": ("const double out_f = exp(a - 0.5 * sq) / sqrt((double)F);", "const double out_f = exp(a - 0.5 * sq);"),
    "fmb_trf_cos_sign": ("dy[d] += g[P + p] * (y[d] * c * co - c * s * W[p * D + d]);",
                         "dy[d] += g[P + p] * (y[d] * c * co + c * s * W[p * D + d]);"),
    "fmb_trf_no_magnitude_term": ("dy[d] += g[p] * (y[d] * c * s + c * co * W[p * D + d]);",
                                  "dy[d] += g[p] * (c * co * W[p * D + d]);"),
    "fmb_elu_derivative": ("dy[d] = g[d] * (y[d] > 0.0 ? 1.0 : exp(y[d]));", "dy[d] = g[d] * (y[d] > 0.0 ? y[d] + 1.0 : exp(y[d]));"),
    "fmb_norm_no_projection": ("dx[d] = (dy[d] - y[d] * ydy) / len;", "dx[d] = dy[d] / len;"),
    "fmb_norm_no_length": ("dx[d] = (dy[d] - y[d] * ydy) / len;", "dx[d] = dy[d] - y[d] * ydy;"),
    "decode_den_uses_k": ("den += oracle_phi1(qh[d]) * zh[d];", "den += oracle_phi1(kh[d]) * zh[d];"),
    "decode_reads_before_update": (
        "        for (int64_t d = 0; d < D; ++d) {\n            double f = oracle_phi1(kh[d]);\n            for (int64_t m = 0; m < M; ++m) Sh[d * M + m] += f * vh[m];\n            zh[d] += f;\n        }\n        double den = 0.0;\n        for (int64_t d = 0; d < D; ++d) den += oracle_phi1(qh[d]) * zh[d];\n        for (int64_t m = 0; m < M; ++m) {\n            double num = 0.0;\n            for (int64_t d = 0; d < D; ++d) num += oracle_phi1(qh[d]) * Sh[d * M + m];\n            oh[m] = num / den;\n        }\n",
        "        double den = 0.0;\n        for (int64_t d = 0; d < D; ++d) den += oracle_phi1(qh[d]) * zh[d];\n        for (int64_t m = 0; m < M; ++m) {\n            double num = 0.0;\n            for (int64_t d = 0; d < D; ++d) num += oracle_phi1(qh[d]) * Sh[d * M + m];\n            oh[m] = num / den;\n        }\n        for (int64_t d = 0; d < D; ++d) {\n            double f = oracle_phi1(kh[d]);\n            for (int64_t m = 0; m < M; ++m) Sh[d * M + m] += f * vh[m];\n            zh[d] += f;\n        }\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mut = tmp_path / f"{name}.c"
    mut.write_text(src.replace(old, new, 1))  # the first site (functions appear in file order)
    lib = oracle.compile_lib(str(mut), str(tmp_path / f"lib{name}.so"))
    fails = oracle_pins.run_all(oracle.Oracle(lib))
    assert fails, f"planted mistake {name} was not caught by any pin"


def test_threads_do_not_change_results():
    rng = np.random.default_rng(3)
    Q, K, V = rng.normal(size=(6, 30, 8)), rng.normal(size=(6, 30, 8)), rng.normal(size=(6, 30, 4))
    a = oracle.causal(Q, K, V, threads=1)
    b = oracle.causal(Q, K, V, threads=4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
