"""Planted mistakes: each plausible slip in the oracle must fail a pin.

Every case copies oracle/oracle.c to a temporary directory, applies one textual
mutation (a dropped term, a wrong sign or index, a transposed operand, a
missing scale), builds it with the same gcc line as the real oracle, routes the
oracle wrapper to that build and runs the pin battery from
test_oracle_pins.py.  The case passes only if at least one pin fails.  This
runs on the CPU only; nothing here touches the GPU library.
"""
import os
import tempfile

import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "diagonal_dropped_from_normaliser": (
        "for (int64_t j = j0; j <= i; ++j) Z += exp(s[j] - m);",
        "for (int64_t j = j0; j < i; ++j) Z += exp(s[j] - m);"),
    "window_one_key_too_many": (
        "return (window > 0 && i - window + 1 > 0) ? i - window + 1 : 0;",
        "return (window > 0 && i - window > 0) ? i - window : 0;"),
    "scale_missing": ("s[j] = scale * dot;", "s[j] = dot;"),
    "scale_squared": ("s[j] = scale * dot;", "s[j] = scale * scale * dot;"),
    "lse_without_max": ("L[i] = m + log(Z);", "L[i] = log(Z);"),
    "lse_log2": ("L[i] = m + log(Z);", "L[i] = m + log2(Z);"),
    "value_row_index": ("acc += p[j] * V[j * D + d];", "acc += p[j] * V[i * D + d];"),
    "key_index_transposed": ("dot += Qi[d] * K[j * D + d];", "dot += Qi[d] * K[i * D + d];"),
    "softmax_jacobian_drops_delta": ("double dS = p[j] * (dp[j] - Delta);",
                                     "double dS = p[j] * dp[j];"),
    "softmax_jacobian_sign": ("double dS = p[j] * (dp[j] - Delta);",
                              "double dS = p[j] * (Delta - dp[j]);"),
    "dq_missing_scale": ("dQ[i * D + d] += scale * dS * K[j * D + d];",
                         "dQ[i * D + d] += dS * K[j * D + d];"),
    "dq_wrong_key_row": ("dQ[i * D + d] += scale * dS * K[j * D + d];",
                         "dQ[i * D + d] += scale * dS * K[i * D + d];"),
    "dk_missing_scale": ("dK[j * D + d] += scale * dS * Q[i * D + d];",
                         "dK[j * D + d] += dS * Q[i * D + d];"),
    "dk_wrong_query_row": ("dK[j * D + d] += scale * dS * Q[i * D + d];",
                           "dK[j * D + d] += scale * dS * Q[j * D + d];"),
    "dv_wrong_grad_row": ("dV[j * D + d] += p[j] * G[i * D + d];",
                          "dV[j * D + d] += p[j] * G[j * D + d];"),
    "dp_uses_keys": ("acc += G[i * D + d] * V[j * D + d];", "acc += G[i * D + d] * K[j * D + d];"),
    "layernorm_unbiased_variance": ("var /= (double)C; /* biased variance */",
                                    "var /= (double)(C - 1);"),
    "layernorm_eps_outside_sqrt": ("double r = 1.0 / sqrt(var + eps);",
                                   "double r = 1.0 / (sqrt(var) + eps);"),
    "layernorm_bwd_drops_mean_term": ("dx[n * C + c] = rstd[n] * (dxh - m1 - xhat[n * C + c] * m2) +",
                                      "dx[n * C + c] = rstd[n] * (dxh - xhat[n * C + c] * m2) +"),
    "heads_interleaved": ("qkv[(b * T + t) * 3 * C + third * C + h * D + d];",
                          "qkv[(b * T + t) * 3 * C + h * 3 * D + third * D + d];"),
    "colsum_skips_the_last_row": ("for (int64_t n = 0; n < N; ++n) acc += x[n * M + j];",
                                  "for (int64_t n = 0; n + 1 < N; ++n) acc += x[n * M + j];"),
    "residual_dropped_in_bwd": ("layer_norm_bwd(du, g, S.xhat, S.rstd, dy, dx, dg, dbl, N, C);",
                                "layer_norm_bwd(du, g, S.xhat, S.rstd, NULL, dx, dg, dbl, N, C);"),
    "decode_cache_in_bhtd_order": ("const double* Kj = kc + ((b * Tmax + j) * H + h) * D;",
                                   "const double* Kj = kc + ((b * H + h) * Tmax + j) * D;"),
    "decode_token_one_position_early": ("const int64_t last = len - 1;  /* the new token's position */",
                                        "const int64_t last = len - 2;"),
    "decode_values_from_keys": ("acc += exp(s[j] - m) / Z * vc[((b * Tmax + j) * H + h) * D + d];",
                                "acc += exp(s[j] - m) / Z * kc[((b * Tmax + j) * H + h) * D + d];"),
    "decode_scale_missing": ("s[j] = dot * scale;", "s[j] = dot;"),
    "decode_lse_without_max": ("lse[bh] = m + log(Z);", "lse[bh] = log(Z);"),
    "rope_rotation_sign": ("Y[i] = r * (X[i] * c - X[i + half] * s);",
                           "Y[i] = r * (X[i] * c + X[i + half] * s);"),
    "rope_adjacent_pairs": ("Y[i + half] = r * (X[i] * s + X[i + half] * c);",
                            "Y[i + half] = r * (X[i] * s + X[i + 1] * c);"),
    "rope_frequency_exponent": ("pow(base, -2.0 * (double)i / (double)D)",
                                "pow(base, -(double)i / (double)D)"),
    "qknorm_sum_not_mean": ("r = gain / sqrt(ss / (double)D + eps);", "r = gain / sqrt(ss + eps);"),
    "qknorm_eps_outside": ("r = gain / sqrt(ss / (double)D + eps);",
                           "r = gain / (sqrt(ss / (double)D) + eps);"),
    "qknorm_bwd_drops_projection": ("dz[d] = gain / rms * G[d] - z[d] * gain / (rms * rms * rms) * m;",
                                    "dz[d] = gain / rms * G[d];"),
    "rope_bwd_not_transposed": ("DX[i] = dz[i] * c + dz[i + half] * s;",
                                "DX[i] = dz[i] * c - dz[i + half] * s;"),
    "philox_key_schedule": ("k1 += 0xBB67AE85u;", "k1 += 0x9E3779B9u;"),
    "philox_word_order": ("const uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;",
                          "const uint32_t y0 = (uint32_t)(p0 >> 32) ^ x1 ^ k0;"),
    "dropout_counter_swapped": ("const uint32_t ctr[4] = {(uint32_t)(j / 8), (uint32_t)i, (uint32_t)bh, 0u};",
                                "const uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(j / 8), (uint32_t)bh, 0u};"),
    "dropout_unscaled": ("w[j] = oracle_dropout_keep(seed, p16, bh0 + bh, i, j) ? w[j] * keep_scale : 0.0;",
                         "w[j] = oracle_dropout_keep(seed, p16, bh0 + bh, i, j) ? w[j] : 0.0;"),
    "dropout_bwd_mask_not_on_dp": ("gw[j] = mk[j] * sum;", "gw[j] = sum;"),
    "weight_grad_transposed": ("for (int64_t c = 0; c < C; ++c) dWp[cp * C + c] += av * dy[n * C + c];",
                               "for (int64_t c = 0; c < C; ++c) dWp[c * C + cp] += av * dy[n * C + c];"),
}

BATTERY = [
    pins.test_golden_forward_worked_example,
    pins.test_golden_backward_worked_example,
    pins.test_single_token_is_identity,
    pins.test_zero_queries_give_running_prefix_mean,
    pins.test_identity_values_expose_the_weight_matrix,
    pins.test_backward_identities,
    lambda: pins.test_against_torch_sdpa_fp64((2, 2, 5, 3)),
    lambda: pins.test_backward_finite_differences_every_element((1, 2, 8, 4)),
    pins.test_sublayer_against_torch_library_ops,
    pins.test_sublayer_finite_differences,
    pins.test_layernorm_output_is_standardised,
    pins.test_layernorm_alone_is_standardised_affine_and_shift_invariant,
    pins.test_layernorm_backward_finite_differences_and_residual,
    pins.test_colsum_of_a_matrix_with_known_column_sums,
    lambda: pins.test_window_against_torch_sdpa_band_mask(3),
    lambda: pins.test_decode_against_torch_sdpa_single_query(3),
    pins.test_decode_closed_forms,
    pins.test_rope_two_columns_is_a_plane_rotation_by_the_position,
    pins.test_rope_four_columns_pairs_and_frequencies,
    lambda: pins.test_qk_norm_against_torch_rms_norm(1.2, 1e-6),
    lambda: pins.test_rope_qknorm_backward_finite_differences(True, True),
    pins.test_philox_known_answer_vectors,
    pins.test_dropout_keep_follows_the_stated_draw_and_rate,
    lambda: pins.test_dropout_against_torch_ops_with_the_same_mask(0.3, 3),
]


def test_unmutated_copy_passes_the_battery(tmp_path):
    out = oracle.compile_source(SRC, str(tmp_path / "liboracle_copy.so"))
    with oracle.use_library(out):
        for pin in BATTERY:
            pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(mutated), str(tmp_path / "liboracle_mutant.so"))
    failed = []
    with oracle.use_library(lib):
        for pin in BATTERY:
            try:
                pin()
            except AssertionError:
                failed.append(getattr(pin, "__name__", "lambda"))
    assert failed, f"planted mistake {name!r} passed every pin"
