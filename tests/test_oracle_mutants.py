"""Planted mistakes in the oracle must turn its pins red.

Each mutant is a copy of oracle.c with one plausible mistake (a dropped
term, a wrong sign or index, a swapped operand, a broken tie rule), built
with gcc into a temporary directory and loaded in a child pytest through
ORACLE_LIB. The child runs the pins named for that mutant and must fail.
Everything here runs on the CPU.
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name: (text in oracle.c, replacement, pin tests that must catch it); the
# text and replacement may be tuples for a mistake that spans two sites.
MUTANTS = {
    "bias_leaks_into_weights": (
        "(double)s[ids[j]] / (sum + eps)", "(double)key[ids[j]] / (sum + eps)",
        ["tests/test_oracle_router.py::test_bias_selects_but_never_weighs"]),
    "eps_dropped": (
        "(double)s[ids[j]] / (sum + eps)", "(double)s[ids[j]] / (sum)",
        ["tests/test_oracle_router.py::test_weights_eps_is_visible_at_tiny_scores"]),
    "routed_scale_on_shared_term": (
        "o[h] += y[h];", "o[h] += L->rsf * y[h];",
        ["tests/test_oracle_experts.py::test_routed_scale_is_linear_and_spares_the_shared_term"]),
    "relu_not_squared": (
        "return r * r;", "return r;",
        ["tests/test_oracle_experts.py::test_activation_special_values"]),
    "gate_up_swapped": (
        "activate(0, proj[i], proj[I + i], L->swiglu_limit)",
        "activate(0, proj[I + i], proj[i], L->swiglu_limit)",
        ["tests/test_oracle_experts.py::test_hand_layer_closed_form"]),
    "silu_sign": (
        "g / (1.0 + exp(-g)) * u", "g / (1.0 + exp(g)) * u",
        ["tests/test_oracle_experts.py::test_activation_special_values"]),
    "ties_to_higher_index": (
        "    return a < b;\n}", "    return a > b;\n}",
        ["tests/test_oracle_router.py::test_topk_exhaustive_small_domain"]),
    "nan_ranks_first": (
        "        return nb;", "        return na;",
        ["tests/test_oracle_router.py::test_topk_exhaustive_small_domain"]),
    "plan_unstable": (
        "    for (int a = 0; a < A; ++a) {\n        int p = fill[ids[a]]++;",
        "    for (int a = A - 1; a >= 0; --a) {\n        int p = fill[ids[a]]++;",
        ["tests/test_oracle_plan.py"]),
    "sigmoid_sign": (
        "1.0f / (1.0f + oracle_exp32(-z))", "1.0f / (1.0f + oracle_exp32(z))",
        ["tests/test_oracle_router.py::test_sigmoid32_closed_form_ln3"]),
    "logit_order_reversed": (
        "        for (int h = h0; h < h1; ++h)\n            p = fmaf",
        "        for (int h = h1 - 1; h >= h0; --h)\n            p = fmaf",
        ["tests/test_oracle_router.py::test_logit_order_is_sequential_fp32_fma"]),
    "logit_in_double": (
        ("        float p = 0.0f;\n        for (int h = h0; h < h1; ++h)",
         "p = fmaf(bf16_value(x_row[h]), w_row[h], p);"),
        ("        double p = 0.0;\n        for (int h = h0; h < h1; ++h)",
         "p += (double)bf16_value(x_row[h]) * (double)w_row[h];"),
        ["tests/test_oracle_router.py::test_logit_order_is_sequential_fp32_fma"]),
    "logit_slice_width_32": (
        "#define ROUTER_SLICE 64", "#define ROUTER_SLICE 32",
        ["tests/test_oracle_router.py::test_logit_slices_and_their_sum_order"]),
    "logit_slice_width_128": (
        "#define ROUTER_SLICE 64", "#define ROUTER_SLICE 128",
        ["tests/test_oracle_router.py::test_logit_slices_and_their_sum_order"]),
    "logit_one_chain": (
        "        float p = 0.0f;\n", "        float p = z;\n        z = 0.0f;\n",
        ["tests/test_oracle_router.py::test_logit_slices_and_their_sum_order"]),
    "logit_slices_summed_backwards": (
        "for (int h0 = 0; h0 < H; h0 += ROUTER_SLICE) {",
        "for (int h0 = (H - 1) / ROUTER_SLICE * ROUTER_SLICE; h0 >= 0; h0 -= ROUTER_SLICE) {",
        ["tests/test_oracle_router.py::test_logit_slices_and_their_sum_order"]),
    "router_weight_transposed": (
        "z[e] = router_logit(x_row, Wr + (size_t)e * H, H);",
        "z[e] = router_logit(x_row, Wr + (size_t)e, H);",
        ["tests/test_oracle_router.py::test_logit_zero_row_and_one_hot_row"]),
    "nibbles_big_endian": (
        "(codes_row[c / 8] >> (4 * (c % 8)))", "(codes_row[c / 8] >> (4 * (7 - c % 8)))",
        ["tests/test_oracle_experts.py::test_affine4_decode_hand_cases"]),
    "affine_group_index": (
        "bf16_value(scale_row[c / group])", "bf16_value(scale_row[c % group])",
        ["tests/test_oracle_experts.py::test_affine4_decode_hand_cases"]),
    "softmax_no_max_shift": (
        "float d = z[e] - m;", "float d = z[e];",
        ["tests/test_oracle_router.py::test_softmax32_exact_points"]),
    "softmax_sum_descending": (
        "    for (int e = 0; e < E; ++e) {\n        float d = z[e] - m;",
        "    for (int e = E - 1; e >= 0; --e) {\n        float d = z[e] - m;",
        ["tests/test_oracle_router.py::test_softmax32_sum_order_constructed"]),
    "softmax_last_term_dropped": (
        "        S = S + s[e];", "        if (e < E - 1)\n            S = S + s[e];",
        ["tests/test_oracle_router.py::test_softmax32_exact_points"]),
    "route_ignores_softmax": (
        "if (score_fn == 1)", "if (score_fn == 2)",
        ["tests/test_oracle_router.py::test_route_softmax_matches_brute_force_and_closed_weights"]),
    "limit_gate_two_sided": (
        "g = (g > limit) ? limit : g;", "g = (g > limit) ? limit : ((g < -limit) ? -limit : g);",
        ["tests/test_oracle_experts.py::test_swiglu_limit_special_values"]),
    "limit_up_one_sided": (
        "u = (u > limit) ? limit : ((u < -limit) ? -limit : u);", "u = (u > limit) ? limit : u;",
        ["tests/test_oracle_experts.py::test_swiglu_limit_special_values"]),
    "limit_skips_shared_expert": (
        "activate(0, proj[i], proj[Is + i], L->swiglu_limit)", "activate(0, proj[i], proj[Is + i], 0.0)",
        ["tests/test_oracle_experts.py::test_swiglu_limit_changes_exactly_the_clamped_tokens"]),
    "norm_eps_dropped": (
        "double inv = 1.0 / sqrt(ss / H + eps);", "double inv = 1.0 / sqrt(ss / H);",
        ["tests/test_oracle_norm.py::test_constant_zero_and_tiny_rows_closed_form"]),
    "norm_mean_over_H_minus_1": (
        "double inv = 1.0 / sqrt(ss / H + eps);", "double inv = 1.0 / sqrt(ss / (H - 1) + eps);",
        ["tests/test_oracle_norm.py::test_one_hot_row_pins_the_mean_and_gamma_index"]),
    "norm_gamma_shifted": (
        "(double)bf16_value(gamma[c]);", "(double)bf16_value(gamma[(c + 1) % H]);",
        ["tests/test_oracle_norm.py::test_one_hot_row_pins_the_mean_and_gamma_index"]),
    "norm_residual_without_h": (
        "res_out[i] = bf16_round(r[c]);", "res_out[i] = res[i];",
        ["tests/test_oracle_norm.py::test_residual_is_the_bf16_of_the_sum_ties_to_even"]),
    "norm_rounding_ties_up": (
        "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))", "if (lower >= 0x8000u)",
        ["tests/test_oracle_norm.py::test_residual_is_the_bf16_of_the_sum_ties_to_even"]),
    "norm_without_sqrt": (
        "double inv = 1.0 / sqrt(ss / H + eps);", "double inv = 1.0 / (ss / H + eps);",
        ["tests/test_oracle_norm.py::test_random_rows_match_the_vector_norm"]),
    "fp8_exponent_bias_8": (
        "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)",
        ["tests/test_oracle_fp8.py::test_e4m3_hand_values"]),
    "fp8_subnormal_scale": (
        "ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)",
        ["tests/test_oracle_fp8.py::test_e4m3_hand_values"]),
    "fp8_no_nan": (
        "    if (e == 15 && m == 7)\n        return NAN;\n", "",
        ["tests/test_oracle_fp8.py::test_e4m3_hand_values"]),
    "fp8_scale_block_transposed": (
        "((size_t)e * (N / 128) + n / 128) * (K / 128);\n        for (int c = 0; c < K; ++c)\n            row[c] = fp8_e4m3_value(codes[c]) * (double)sc[c / 128];",
        "(size_t)e * (N / 128) * (K / 128) + n / 128;\n        for (int c = 0; c < K; ++c)\n            row[c] = fp8_e4m3_value(codes[c]) * (double)sc[(c / 128) * (N / 128)];",
        ["tests/test_oracle_fp8.py::test_fp8_layer_matches_dense_float64"]),
    "fp4_high_nibble_first": (
        "return (row[c / 2] >> (4 * (c % 2))) & 15u;", "return (row[c / 2] >> (4 * (1 - c % 2))) & 15u;",
        ["tests/test_oracle_nvfp4.py::test_packing_is_low_nibble_first"]),
    "fp4_exponent_bias_0": (
        "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)",
        ["tests/test_oracle_nvfp4.py::test_e2m1_hand_values"]),
    "nvfp4_group_32": (
        "fp8_e4m3_value(sc[c / 16]) * g;", "fp8_e4m3_value(sc[c / 32]) * g;",
        ["tests/test_oracle_nvfp4.py::test_nvfp4_layer_matches_dense_float64"]),
    "nvfp4_global_dropped": (
        "fp8_e4m3_value(sc[c / 16]) * g;", "fp8_e4m3_value(sc[c / 16]);",
        ["tests/test_oracle_nvfp4.py::test_hand_layer"]),
    "mxfp4_group_16": (
        "e8m0_value(sc[c / 32]);", "e8m0_value(sc[c / 16]);",
        ["tests/test_oracle_nvfp4.py::test_mxfp4_layer_matches_dense_float64"]),
    "e8m0_bias_128": (
        "ldexp(1.0, (int)b - 127);", "ldexp(1.0, (int)b - 128);",
        ["tests/test_oracle_nvfp4.py::test_e8m0_hand_values"]),
    "e8m0_no_nan": (
        "return b == 0xFF ? NAN : ldexp", "return b == 0x1FF ? NAN : ldexp",
        ["tests/test_oracle_nvfp4.py::test_e8m0_hand_values"]),
    "round_h_ignored": (
        "return L->round_h ? (double)bf16_value(bf16_round((float)h)) : h;", "return h;",
        ["tests/test_oracle_round_h.py::test_round_h_hand_values_routed_and_shared"]),
    "round_h_truncates": (
        "return L->round_h ? (double)bf16_value(bf16_round((float)h)) : h;",
        "float f = (float)h; uint32_t b; memcpy(&b, &f, 4); b &= 0xFFFF0000u; memcpy(&f, &b, 4);\n"
        "    return L->round_h ? (double)f : h;",
        ["tests/test_oracle_round_h.py::test_round_h_hand_values_routed_and_shared"]),
    "round_h_shared_skipped": (
        "proj[i] = stored_h(L, (L->act == 0) ? activate(0, proj[i], proj[Is + i], L->swiglu_limit)",
        "proj[i] = ((L->act == 0) ? activate(0, proj[i], proj[Is + i], L->swiglu_limit)",
        ["tests/test_oracle_round_h.py::test_round_h_hand_values_routed_and_shared"]),
    "mimic_combine_descending": (
        "            for (int j = 0; j < k; ++j) {\n                float wj = w[",
        "            for (int j = k - 1; j >= 0; --j) {\n                float wj = w[",
        ["tests/test_oracle_mimic.py::test_combine_is_an_fma_chain_over_j_ascending"]),
    "mimic_combine_unfused": (
        "acc = fmaf(wj, y[((size_t)t * k + j) * H + h], acc);",
        "acc = wj * y[((size_t)t * k + j) * H + h] + acc;",
        ["tests/test_oracle_mimic.py::test_combine_is_an_fma_chain_over_j_ascending"]),
    "mimic_shared_before_scale": (
        "            if (!fold)\n                acc = acc * rsf;\n            if (shared)\n"
        "                acc = acc + shared[(size_t)t * H + h];",
        "            if (shared)\n                acc = acc + shared[(size_t)t * H + h];\n"
        "            if (!fold)\n                acc = acc * rsf;",
        ["tests/test_oracle_mimic.py::test_routed_scale_once_after_the_sum_and_shared_unscaled"]),
    "mimic_always_folded": (
        ("                if (fold)\n                    wj = rsf * wj;",
         "            if (!fold)\n                acc = acc * rsf;\n"),
        ("                wj = rsf * wj;", ""),
        ["tests/test_oracle_mimic.py::test_routed_scale_once_after_the_sum_and_shared_unscaled"]),
    "mimic_epilogue_truncates": (
        "        return bf16_round(r * r);",
        "        float q = r * r;\n        uint32_t b;\n        memcpy(&b, &q, 4);\n"
        "        return (uint16_t)(b >> 16);",
        ["tests/test_oracle_mimic.py::test_epilogue_rounding_ties_to_even_by_exact_arithmetic"]),
    "mimic_relu_by_fmax": (
        "float r = (u < 0.0f) ? 0.0f : u;\n        return bf16_round",
        "float r = fmaxf(u, 0.0f);\n        return bf16_round",
        ["tests/test_oracle_mimic.py::test_epilogue_relu2_special_values_and_rounding"]),
    "mimic_swiglu_gate_up_swapped": (
        "bf16_round((g * oracle_sigmoid32(g)) * u)", "bf16_round((u * oracle_sigmoid32(u)) * g)",
        ["tests/test_oracle_mimic.py::test_epilogue_saturated_swiglu_is_the_product"]),
    "exp_taylor_term_dropped": (
        "    p = fmaf(p, r, 1.0f / 6.0f);        /* 1/3! */\n", "",
        ["tests/test_oracle_router.py::test_exp32_sweep_against_libm"]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_killed(name, tmp_path):
    old, new, pins = MUTANTS[name]
    src = open(O.SOURCE).read()
    olds, news = (old, new) if isinstance(old, tuple) else ((old,), (new,))
    for o, n in zip(olds, news):
        assert src.count(o) == 1, f"mutation site for {name} not unique"
        src = src.replace(o, n)
    mut_src = tmp_path / "oracle_mut.c"
    mut_src.write_text(src)
    lib = O.compile_source(str(mut_src), str(tmp_path / "liboracle_mut.so"), werror=False)
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *pins], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"mutant {name} survived:\n{r.stdout[-2000:]}"
