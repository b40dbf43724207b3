"""The oracle's pins must catch plausible mistakes.

Each case below plants one slip in a copy of the oracle's C source (on the
CPU, in a temporary directory), builds it, points the oracle binding at the
broken copy and runs the pin tests from test_oracle.py against it: at least
one pin must fail.  The real oracle is restored afterwards.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "convrot_oracle.c")

MUTANTS = [
    ("ties_to_even", "static double round_half_away(double v) { return round(v); }",
     "static double round_half_away(double v) { return rint(v); }"),
    ("no_normalisation", "double norm = 1.0 / sqrt((double)g);", "double norm = 1.0;"),
    ("wrong_hadamard_or", "(__builtin_popcount((unsigned)(i & j)) & 1)",
     "(__builtin_popcount((unsigned)(i | j)) & 1)"),
    ("permuted_columns", "acc += in[base + i] * H[(int64_t)i * g + j];",
     "acc += in[base + i] * H[(int64_t)i * g + ((j + 1) % g)];"),
    ("interleaved_groups", "out[base + j] = acc;", "out[base / g + (int64_t)j * (K / g)] = acc;"),
    ("scale_over_128", "float s = (float)(amax / 127.0);", "float s = (float)(amax / 128.0);"),
    ("max_not_absmax", "double a = fabs(v[k]);", "double a = v[k];"),
    ("forgot_rotation_activations", "quantize_row_i8(rot, K, xq + m * K, x_scale + m);",
     "quantize_row_i8(in, K, xq + m * K, x_scale + m);"),
    ("forgot_rotation_weights", "quantize_row_i8(rot, K, wq + n * K, scale + n);",
     "quantize_row_i8(in, K, wq + n * K, scale + n);"),
    ("rotation_rounded_to_fp32", "            rotate_row_f64(in, K, g, H, rot);\n            quantize_row_i8(rot, K, xq",
     "            rotate_row_f64(in, K, g, H, rot);\n"
     "            for (int64_t k = 0; k < K; ++k) rot[k] = (double)(float)rot[k];\n"
     "            quantize_row_i8(rot, K, xq"),
    ("quotient_rounded_to_fp32", "double r = round_half_away(v[k] / (double)s);\n        if (r > 127.0)",
     "double r = round_half_away((double)(float)(v[k] / (double)s));\n        if (r > 127.0)"),
    ("transposed_weight", "(int64_t)wq[n * K + k];", "(int64_t)wq[k * N + n];"),
    ("epilogue_order", "float t = a * x_scale[m];\n            float r = t * w_scale[n];",
     "float t = x_scale[m] * w_scale[n];\n            float r = a * t;"),
    ("bf16_truncation", "if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))\n        kept += 1u;",
     "(void)dropped;"),
    ("nibble_order", "(uint8_t)(lo | (hi << 4));", "(uint8_t)(hi | (lo << 4));"),
    ("int4_clamp_8", "if (r > 7.0) r = 7.0;", "if (r > 8.0) r = 8.0;"),
    ("int4_divisor_8", "(double)(100 - i) / 700.0", "(double)(100 - i) / 800.0"),
    ("no_sign_extension", "(int8_t)(lo >= 8 ? lo - 16 : lo);", "(int8_t)(lo);"),
    ("int4_no_search", "for (int i = 0; i <= 50; ++i) {", "for (int i = 0; i <= 0; ++i) {"),
    ("int4_ties_to_smaller_c", "(i == 0 || e < best_err)", "(i == 0 || e <= best_err)"),
    ("int4_forced_index_ignored", "const int take = force_index ? (i == force_index[n])",
     "const int take = 0 ? (i == force_index[n])"),
    ("amax_first_group_only", "    for (int64_t k = 0; k < K; ++k) {\n        double a = fabs(v[k]);",
     "    for (int64_t k = 0; k < (K < 256 ? K : 256); ++k) {\n        double a = fabs(v[k]);"),
    ("int4_amax_unrotated", "if (fabs(rot[k]) > amax) amax = fabs(rot[k]);",
     "if (fabs(in[k]) > amax) amax = fabs(in[k]);"),
    ("rmsnorm_w_not_one_plus_w", "const float u = t * (1.0f + w[k]);", "const float u = t * w[k];"),
    ("rmsnorm_sum_not_mean", "const float ms = (float)(ss / (double)K);", "const float ms = (float)ss;"),
    ("rmsnorm_no_root", "const float r = 1.0f / sqrtf(ms + eps);", "const float r = 1.0f / (ms + eps);"),
    ("rmsnorm_eps_outside_root", "const float r = 1.0f / sqrtf(ms + eps);",
     "const float r = 1.0f / (sqrtf(ms) + eps);"),
    ("rmsnorm_mean_abs", "ss += v * v;", "ss += fabs(v) * fabs(v) * (v < 0 ? 0.5 : 1.0);"),
    ("dequant_no_scale", "const double s = (double)w_scale[n];", "const double s = 1.0;"),
    ("dequant_skips_rotation", "t += (H[(int64_t)j * g + k] > 0.0 ? 1.0 : -1.0) * (double)q[base + j];",
     "t += (j == k ? 1.0 : 0.0) * (double)q[base + j];"),
    ("dequant_rows_swapped", "const double s = (double)w_scale[n];", "const double s = (double)w_scale[N - 1 - n];"),
    ("dequant_sign_transposed_block", "t += (H[(int64_t)j * g + k] > 0.0 ? 1.0 : -1.0) * (double)q[base + j];",
     "t += (H[(int64_t)j * g + ((k + 1) % g)] > 0.0 ? 1.0 : -1.0) * (double)q[base + j];"),
    ("dequant_dense_rounded_terms",
     "                double t = 0.0;\n                for (int j = 0; j < g; ++j)\n"
     "                    t += (H[(int64_t)j * g + k] > 0.0 ? 1.0 : -1.0) * (double)q[base + j];\n"
     "                const double u = (t * s) * norm + 0.0;",
     "                double u = 0.0;\n                for (int j = 0; j < g; ++j)\n"
     "                    u += ((double)q[base + j] * s) * H[(int64_t)j * g + k];\n                (void)norm;"),
    ("dequant_negative_zero", "const double u = (t * s) * norm + 0.0;", "const double u = (t * s) * norm;"),
    ("gemm_bf16_drops_last_k", "for (int64_t k = 0; k < K; ++k)\n                acc += bf16_bits_to_double",
     "for (int64_t k = 0; k + 1 < K; ++k)\n                acc += bf16_bits_to_double"),
    ("gemm_bf16_fp32_accumulation", "double acc = 0.0;\n            for (int64_t k = 0; k < K; ++k)\n                acc += bf16",
     "float acc = 0.0f;\n            for (int64_t k = 0; k < K; ++k)\n                acc += bf16"),
]

PIN_TESTS = [
    "test_hadamard_is_scipy_sylvester", "test_hadamard_orthogonal_bit_exact",
    "test_rotation_matches_blockwise_library_product", "test_rotation_groups_are_contiguous",
    "test_rotation_one_hot_closed_form", "test_worked_one_hot", "test_worked_constant_group",
    "test_worked_half_away_ties_rotated", "test_worked_identity_group_ties",
    "test_worked_quotient_decided_in_fp64", "test_worked_rotation_kept_in_fp64",
    "test_codes_range_and_absmax_code", "test_scale_is_absmax_over_127",
    "test_rotate_quant_brute_force_tiny", "test_quantize_weight_i8_brute_force_tiny",
    "test_gemm_exact_vs_int64_matmul", "test_epilogue_vs_torch_bf16_cast",
    "test_epilogue_order_and_bf16_ties", "test_epilogue_multiplies_token_scale_first",
    "test_rotation_suppresses_outlier_error",
    "test_unpack_all_256_bytes", "test_worked_nibble_order", "test_worked_int4_equal_magnitude",
    "test_int4_clip_search_brute_force", "test_int4_forced_candidate", "test_int4_clip_ties_keep_the_larger_c",
    "test_rmsnorm_constant_power_of_two_rows", "test_rmsnorm_one_hot_gives_sqrt_k",
    "test_rmsnorm_weight_enters_as_one_plus_w", "test_rmsnorm_eps_inside_the_root",
    "test_rmsnorm_zero_row_and_unit_rms",
    "test_dequant_one_hot_closed_form", "test_dequant_group_one_is_scale_times_code",
    "test_dequant_exact_zeros_are_positive_zero",
    "test_dequant_inverts_quantize_within_bound", "test_dequant_int4_error_is_the_clip_search_error",
    "test_gemm_bf16_brute_force_tiny", "test_gemm_bf16_identity_and_rounding_order",
    "test_gemm_bf16_sum_carries_fp64",
]


def _run_pin(name):
    """Run one pin as pytest would: every parameter set of its parametrize
    mark (tests drawn by hypothesis generate their own arguments)."""
    fn = getattr(pins, name)
    import inspect
    params = inspect.signature(fn).parameters
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if marks:
        argnames, argvalues = marks[0].args[0], marks[0].args[1]
        names = [a.strip() for a in argnames.split(",")] if isinstance(argnames, str) else list(argnames)
        for vals in argvalues:
            vals = vals if len(names) > 1 else (vals,)
            kwargs = dict(zip(names, vals))
            if "oracle_mod" in params:
                kwargs["oracle_mod"] = oracle
            fn(**kwargs)
    elif "oracle_mod" in params:
        fn(oracle)
    else:
        fn()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_kill_mutant(name, old, new):
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found in the oracle source"
    with tempfile.TemporaryDirectory() as d:
        csrc = os.path.join(d, "m.c")
        lib = os.path.join(d, f"liboracle_{name}.so")
        with open(csrc, "w") as f:
            f.write(src.replace(old, new))
        subprocess.run(["gcc", *oracle.CFLAGS, "-w", csrc, "-o", lib, "-lm"], check=True)
        oracle.use_library(lib)
        try:
            killed_by = None
            for t in PIN_TESTS:
                try:
                    _run_pin(t)
                except Exception as e:  # any failure of a pin kills the mutant
                    killed_by = f"{t}: {type(e).__name__}"
                    break
        finally:
            oracle.use_library(None)
    assert killed_by is not None, f"no pin detects mutant {name}"
