"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a copy of ``oracle/oracle.c`` (a
dropped term, a wrong sign, a swapped index or constant), builds that copy
with the same compiler flags, and requires that at least one pin in
``tests/pins.py`` rejects it.  The real oracle is never modified.
"""
import os

import pytest

import oracle
from pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "softmax_den_without_max": ("den += exp(xr[j] - m);", "den += exp(xr[j]);"),
    "softmax_exp_sign": ("yr[j] = exp(xr[j] - m) / den;", "yr[j] = exp(m - xr[j]) / den;"),
    "row_max_is_min": ("if (x[j] > m)\n            m = x[j];", "if (x[j] < m || m == -INFINITY)\n            m = x[j];"),
    "online_rescale_dropped": ("return exp(m_old - m_new);", "return 1.0;"),
    "online_rescale_inverted": ("return exp(m_old - m_new);", "return exp(m_new - m_old);"),
    "online_block_sum_old_max": ("block_sum += exp(x[j] - m_new);", "block_sum += exp(x[j] - block_max);"),
    "stats_neg_inf_guard_dropped": ("    if (m != -INFINITY)\n        for (int64_t j = 0; j < N; ++j)\n            d += exp(x[j] - m);", "    for (int64_t j = 0; j < N; ++j)\n        d += exp(x[j] - m);"),
    "online_neg_inf_guard_dropped": ("        if (m_new != -INFINITY)\n            for (int64_t j = s; j < e; ++j)", "        for (int64_t j = s; j < e; ++j)"),
    "merge_second_unscaled": ("d1 * rescale(m1, M) + d2 * rescale(m2, M)", "d1 * rescale(m1, M) + d2"),
    "split_chunk_size": ("int64_t C = (N + S - 1) / S;\n    double m = -INFINITY", "int64_t C = N / S + 1;\n    double m = -INFINITY"),
    "gelu_cubic_coeff": ("0.044715 * z * z * z", "0.04715 * z * z * z"),
    "gelu_half_dropped": ("return 0.5 * z * (1.0 + tanh(", "return z * (1.0 + tanh("),
    "gelu_scale_constant": ("sqrt(2.0 / M_PI)", "sqrt(M_PI / 2.0)"),
    "gelu_cubic_sign": ("(z + 0.044715 * z * z * z)", "(z - 0.044715 * z * z * z)"),
    "ln_unbiased_variance": ("double var = q / (double)N;", "double var = q / (double)(N > 1 ? N - 1 : 1);"),
    "ln_eps_outside_sqrt": ("*rstd_out = 1.0 / sqrt(var + eps);", "*rstd_out = 1.0 / (sqrt(var) + eps);"),
    "ln_eps_dropped": ("*rstd_out = 1.0 / sqrt(var + eps);", "*rstd_out = 1.0 / sqrt(var);"),
    "ln_bias_sign": ("* rstd * w[j] + b[j];\n            yr[j] = oracle_gelu_tanh(z);", "* rstd * w[j] - b[j];\n            yr[j] = oracle_gelu_tanh(z);"),
    "ln_weight_dropped": ("* rstd * w[j] + b[j];\n            yr[j] = oracle_gelu_tanh(z);", "* rstd + b[j];\n            yr[j] = oracle_gelu_tanh(z);"),
    "ex_bias_sign": ("* rstd * w[j] + b[j];\n            if (gelu == 2)", "* rstd * w[j] - b[j];\n            if (gelu == 2)"),
    "ln_mean_divisor": ("double mean = s / (double)N;", "double mean = s / (double)(N + 1);"),
    "ln_var_uncentered": ("q += (x[j] - mean) * (x[j] - mean);\n    double var", "q += x[j] * x[j];\n    double var"),
    "chunk_mean_divisor": ("double mean = s / (double)n;", "double mean = s / (double)(n + 1);"),
    "rms_sum_not_mean": ("double ms = q / (double)N;", "double ms = q;"),
    "rms_eps_outside_sqrt": ("*inv_out = 1.0 / sqrt(ms + eps);", "*inv_out = 1.0 / (sqrt(ms) + eps);"),
    "rms_centred": ("        q += x[j] * x[j];\n    double ms", "        q += (x[j] - x[0]) * (x[j] - x[0]);\n    double ms"),
    "rms_weight_dropped": ("y[i * N + j] = x[i * N + j] * inv * w[j];", "y[i * N + j] = x[i * N + j] * inv;"),
    "residual_sign": ("rr[j] = x[i * N + j] + res[i * N + j];", "rr[j] = x[i * N + j] - res[i * N + j];"),
    "residual_not_normalized": ("y[i * N + j] = rr[j] * inv * w[j];", "y[i * N + j] = x[i * N + j] * inv * w[j];"),
    "gelu_erf_no_sqrt2": ("erf(z / sqrt(2.0))", "erf(z)"),
    "gelu_erf_half_dropped": ("return 0.5 * z * (1.0 + erf(", "return z * (1.0 + erf("),
    "chunk_m2_uncentred": ("        q += (x[j] - mean) * (x[j] - mean);\n    *mean_out = mean;", "        q += x[j] * x[j];\n    *mean_out = mean;"),
    "chan_delta_term_dropped": ("*m2_out = m2_1 + m2_2 + delta * delta * n1 * n2 / n;", "*m2_out = m2_1 + m2_2;"),
    "chan_mean_weight": ("*mean_out = mean1 + delta * n2 / n;", "*mean_out = mean1 + delta * n1 / n;"),
    "chan_identity_swapped": ("*n_out = n2, *mean_out = mean2, *m2_out = m2_2;", "*n_out = n1, *mean_out = mean1, *m2_out = m2_1;"),
    "split_var_divisor": ("rstd = 1.0 / sqrt(m2 / (double)N + eps);", "rstd = 1.0 / sqrt(m2 / (double)(N - 1) + eps);"),
    "ex_gelu_kind_ignored": ("yr[j] = gelu ? oracle_gelu_erf(z) : oracle_gelu_tanh(z);", "yr[j] = oracle_gelu_tanh(z);"),
    "ex_plain_layernorm_activated": ("            if (gelu == 2)\n                yr[j] = z;", "            if (gelu == 2)\n                yr[j] = oracle_gelu_tanh(z);"),
    "row_sum_drops_last": ("        for (int64_t j = 0; j < N; ++j)\n            s += x[i * N + j];", "        for (int64_t j = 0; j + 1 < N; ++j)\n            s += x[i * N + j];"),
    "row_sum_first_twice": ("        double s = 0.0;\n        for (int64_t j = 0; j < N; ++j)\n            s += x[i * N + j];", "        double s = x[i * N];\n        for (int64_t j = 0; j < N; ++j)\n            s += x[i * N + j];"),
    "row_max_ignores_nan": ("        if (isnan(x[j]))\n            return NAN;\n", ""),
    "attn_scale_dropped": ("                s[j] = dot * scale;", "                s[j] = dot;"),
    "attn_causal_off_by_one": ("int64_t n = causal ? i + 1 : T;", "int64_t n = causal ? (i > 0 ? i : 1) : T;"),
    "attn_causal_ignored": ("int64_t n = causal ? i + 1 : T;", "int64_t n = T;"),
    "attn_no_max_shift": ("                w[j] = exp(s[j] - m);\n", "                w[j] = exp(s[j]);\n"),
    "attn_unnormalized": ("                oh[i * d + c] = acc / den;", "                oh[i * d + c] = acc;"),
    "attn_key_index": ("dot += qh[i * d + c] * kh[j * d + c];\n                s[j]", "dot += qh[i * d + c] * kh[i * d + c];\n                s[j]"),
    "flash_acc_not_rescaled": ("                        acc[r * d + c] *= alpha;", ""),
    "flash_l_not_rescaled": ("l[r] = alpha * l[r] + psum;", "l[r] = l[r] + psum;"),
    "flash_causal_strict": ("sblk[t] = (causal && j > i) ? -INFINITY", "sblk[t] = (causal && j >= i && j > 0) ? -INFINITY"),
    "flash_alpha_inverted": ("double alpha = m[r] == -INFINITY ? 0.0 : exp(m[r] - m_new);", "double alpha = m[r] == -INFINITY ? 0.0 : exp(m_new - m[r]);"),
    "apply_without_max": ("y[j] = exp(x[j] - m) / d;", "y[j] = exp(x[j]) / d;"),
    "attn_rows_position_ignored": ("int64_t n = causal ? pos[r] + 1 : T;", "int64_t n = causal ? r + 1 : T;"),
    "attn_rows_query_row": ("dot += q[r * d + c] * k[j * d + c];", "dot += q[c] * k[j * d + c];"),
    "split_moments_chunk_floor": ("    int64_t C = (N + S - 1) / S;\n    double n = 0.0", "    int64_t C = N / S;\n    if (C < 1)\n        C = 1;\n    double n = 0.0"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(str(tmp_path / "libmutant.so"), str(path))
    mutant = oracle.Oracle(lib)
    failed = []
    for check in PINS:
        try:
            check(mutant)
        except (AssertionError, FloatingPointError, ValueError, OverflowError, ZeroDivisionError):
            failed.append(check.__name__)
    assert failed, f"no pin rejects the mutant {name}"
