"""The pins catch plausible mistakes: each case below plants one mistake in a
copy of the oracle's C source, builds it on the CPU, routes the oracle binding
to it, and requires at least one pin test to fail.  The real oracle is never
modified."""
import os
import subprocess

import pytest

from oracle import oracle as O
import test_oracle_codecs as TC
import test_oracle_four_over_six as T46
import test_oracle_scale_domains as TD
import test_oracle_single_pass as TS
import test_oracle_quantize as TQ
import test_oracle_route_gemm as TR

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "nvfp4_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("outer_scale_divisor", "float s_g = amax / 2688.0f;", "float s_g = amax / 2687.0f;"),
    ("block_target_code", "quantize_block(x + b * 16, s_g, 6.0f, c)", "quantize_block(x + b * 16, s_g, 4.0f, c)"),
    ("nibble_order", "codes[e / 2] |= (uint8_t)((e % 2) ? (code << 4) : code);",
     "codes[e / 2] |= (uint8_t)((e % 2) ? code : (code << 4));"),
    ("e2m1_ties_to_odd", "(dist == best_dist && (i % 2u) == 0u && (best % 2u) != 0u)",
     "(dist == best_dist && (i % 2u) != 0u && (best % 2u) == 0u)"),
    ("e4m3_ties_to_odd", "(dist == best_dist && (b % 2u) == 0u)", "(dist == best_dist && (b % 2u) != 0u)"),
    ("e4m3_subnormal_step", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("e4m3_bias", "v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);", "v = ldexp(1.0 + (double)m / 8.0, (int)e - 8);"),
    ("block_max_half_block", "  for (int i = 0; i < 16; ++i) {\n    float a = fabsf(orc_bf16_to_f32(blk[i]));",
     "  for (int i = 0; i < 8; ++i) {\n    float a = fabsf(orc_bf16_to_f32(blk[i]));"),
    ("no_underflow_guard", "if (d == 0.0f) {", "if (0) {"),
    ("sign_dropped", "if (signbit(xv)) code |= 8u; else code &= 7u;", "code &= 7u;"),
    ("reciprocal_instead_of_division", "float r = xv / d;", "float r = xv * (1.0f / d);"),
    ("amax_in_ignored", "float amax = amax_in ? amax_in[r] : orc_row_amax(xr, k);",
     "float amax = orc_row_amax(xr, k);"),
    ("group_amax_first_row_only", "for (int64_t r = r0; r < r1; ++r) {\n    float a = orc_row_amax",
     "for (int64_t r = r0; r < r0 + 1; ++r) {\n    float a = orc_row_amax"),
    ("dot_drops_first_term", "for (int64_t i = 0; i < k; ++i) {\n    double p = a[i] * b[i];",
     "for (int64_t i = 1; i < k; ++i) {\n    double p = a[i] * b[i];"),
    ("gemm_wrong_group_weights", "orc_dequantize_row(b_codes + ((int64_t)g * n + j) * (k / 2),\n"
     "                         b_scales + ((int64_t)g * n + j) * (k / 16), 1.0f, k, bdec + j * k);\n"
     "    double sgb",
     "orc_dequantize_row(b_codes + ((int64_t)j) * (k / 2),\n"
     "                         b_scales + ((int64_t)j) * (k / 16), 1.0f, k, bdec + j * k);\n"
     "    double sgb"),
    ("gemm_drops_weight_scale", "out[r * n + j] = (float)(s * sga * sgb);", "out[r * n + j] = (float)(s * sga);"),
    ("route_unstable_order", "int64_t r = offsets[e] + fill[e];", "int64_t r = offsets[e] + counts[e] - 1 - fill[e];"),
    ("route_ignores_align", "int64_t padded = (counts[e] + align - 1) / align * align;", "int64_t padded = counts[e];"),
    ("swiglu_gate_up_swapped", "double g = (double)c[r * 2 * inter + j];\n      double u = (double)c[r * 2 * inter + inter + j];",
     "double u = (double)c[r * 2 * inter + j];\n      double g = (double)c[r * 2 * inter + inter + j];"),
    ("swiglu_drops_router_weight", "silu * u * (double)prob[r]", "silu * u"),
    ("combine_skips_first_slot", "for (int32_t j = 0; j < topk; ++j) {\n        int32_t r = dst_row",
     "for (int32_t j = 1; j < topk; ++j) {\n        int32_t r = dst_row"),
    ("bf16_ties_to_odd", "(dist == best_dist && (c & 1u) == 0u)", "(dist == best_dist && (c & 1u) != 0u)"),
    ("tile_max_first_row_only", "for (int64_t r = t0; r < t0 + 16; ++r) {\n            float a = orc_row_amax",
     "for (int64_t r = t0; r < t0 + 1; ++r) {\n            float a = orc_row_amax"),
    ("tile_scale_from_own_row", "quantize_block_bmax(x + r * ld_x + b * 16, tmax, s_g, 6.0f, c)",
     "quantize_block(x + r * ld_x + b * 16, s_g, 6.0f, c)"),
    ("four_six_ties_pick_four", "int four = e4 < e6;", "int four = e4 <= e6;"),
    ("four_six_outer_divisor", "float s_g = amax / 1536.0f;", "float s_g = amax / 1792.0f;"),
    ("four_six_metrics_swapped", "float term = (metric == 1) ? e * e : fabsf(e);",
     "float term = (metric == 1) ? fabsf(e) : e * e;"),
    ("four_six_second_top", "quantize_block(blk, s_g, 4.0f, c4)", "quantize_block(blk, s_g, 3.0f, c4)"),
    ("four_six_error_without_outer_scale", "float v = qs * s_g;", "float v = qs;"),
    ("online_amax_not_running", "if (rowmax > gamax) gamax = rowmax;", "gamax = rowmax;"),
    ("online_scale_before_tile_max", "if (rowmax > gamax) gamax = rowmax;\n      float s = gamax / 2688.0f;",
     "float s = gamax / 2688.0f;\n      if (rowmax > gamax) gamax = rowmax;"),
    ("online_rescale_dropped", "o = o * (gs_prev / gsi) + d_o;", "o = o + d_o;"),
    ("online_rescale_inverted", "o = o * (gs_prev / gsi) + d_o;", "o = o * (gsi / (gs_prev + 1e-30)) + d_o;"),
    ("online_final_scale_first_tile", "out[r * n + j] = (float)(o * gs_prev * sgw);",
     "out[r * n + j] = (float)(o * (double)gsr[0] * sgw);"),
    ("online_tile_end_off_by_one", "const int64_t c0 = i * tile, c1 = (c0 + tile < inter) ? c0 + tile : inter;\n      float rowmax",
     "const int64_t c0 = i * tile, c1 = (c0 + tile < inter) ? c0 + tile - 16 : inter;\n      float rowmax"),
    ("online_zero_tile_not_skipped", "if (gsi == 0.0) continue;", "if (gsi < 0.0) continue;"),
    ("four_six_last_element_dropped", "  for (int i = 0; i < 16; ++i) {\n    float xv = orc_bf16_to_f32(blk[i]);\n    float qs",
     "  for (int i = 0; i < 15; ++i) {\n    float xv = orc_bf16_to_f32(blk[i]);\n    float qs"),
]

# cheap pins first; each mutant stops at the first pin that fails
PINS = [
    TQ.test_hand_worked_row, TQ.test_hand_worked_tie_row, TQ.test_zero_rows, TQ.test_sign_symmetry,
    TQ.test_lattice_points_quantize_to_themselves, TQ.test_amax_in_is_the_outer_scale_domain,
    TQ.test_group_domain_is_row_domain_with_the_group_amax, TC.test_e2m1_encode_sign_of_zero_and_negatives,
    TC.test_e4m3_decode_matches_torch_float8_e4m3fn, TR.test_route_matches_numpy_stable_sort,
    TR.test_gemm_matches_numpy_matmul_of_dequantized_operands, TR.test_gemm_one_hot_rows_give_single_products,
    TR.test_swiglu_is_nearest_bf16_of_fp64_silu_product, TR.test_combine_matches_numpy_gather_sum,
    TC.test_e2m1_encode_is_round_to_nearest_even_on_grid, TC.test_f64_to_bf16_matches_torch_for_binary32_values,
    TC.test_e4m3_encode_matches_torch_cast_below_448,
    T46.test_hand_worked_four_over_six_row, T46.test_four_over_six_zero_and_sign_rows,
    T46.test_six_candidate_is_the_standard_quantizer_at_175_amax_and_choice_minimises_error,
    TD.test_2d_quantization_is_transpose_consistent,
    TD.test_2d_tile_scale_is_the_1d_scale_of_the_row_holding_the_tile_maximum,
    TS.test_hand_worked_three_tile_row, TS.test_zero_rows_give_zero,
    TS.test_tile_scales_are_the_running_maximum,
]


@pytest.mark.parametrize("name,orig,mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, mutant, tmp_path):
    with open(SRC) as f:
        src = f.read()
    assert src.count(orig) == 1, f"mutation site for {name} not found exactly once"
    mdir = tmp_path / name
    mdir.mkdir()
    csrc = mdir / "nvfp4_oracle.c"
    csrc.write_text(src.replace(orig, mutant))
    hdr = os.path.join(os.path.dirname(SRC), "nvfp4_oracle.h")
    (mdir / "nvfp4_oracle.h").write_text(open(hdr).read())
    so = mdir / "liboracle_mutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                    "-fPIC", "-shared", "-o", str(so), str(csrc), "-lm"], check=True)
    O.use_library(str(so))
    caught = None
    try:
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught = pin.__name__
                break
    finally:
        O.use_library(None)
    assert caught is not None, f"planted mistake {name} passed every pin"
