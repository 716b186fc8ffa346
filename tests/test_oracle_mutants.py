"""Plant plausible mistakes in a copy of the oracle's C source (on the CPU)
and check that the pins in test_oracle_pins.py catch every one of them.

The mutated copies are built into a temporary directory; the real oracle
library is restored after each case.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from oracle import oracle as omod

import test_oracle_pins as pins

SRC = open(obuild.SRC).read()

# (name, original text, planted mistake, pins expected to fail at least once)
MUTANTS = [
    ("no_inv_sqrt_b", "*s = step * oracle_inv_sqrt_b(b);", "*s = step;",
     ["test_golden_hand_example_b4", "test_rotation_identity_end_to_end"]),
    ("butterfly_sign", "blk[i + h] = a - c;", "blk[i + h] = c - a;",
     ["test_fwht_columns_are_sylvester", "test_golden_hand_example_b4"]),
    ("truncating_round", "float t = rintf(v[k] * inv);", "float t = truncf(v[k] * inv);",
     ["test_golden_hand_example_b4", "test_rowquant_rne_ties"]),
    ("round_half_away", "float t = rintf(v[k] * inv);", "float t = roundf(v[k] * inv);",
     ["test_rowquant_rne_ties", "test_b1_is_textbook_w8a8"]),
    ("grid_128", "float inv = 127.0f / amax;", "float inv = 128.0f / amax;",
     ["test_golden_hand_example_b4", "test_rowquant_invariants"]),
    ("transposed_weight", "const int8_t *w = qw + n * K;", "const int8_t *w = qw + n;",
     ["test_gemm_brute_force_tiny", "test_golden_hand_example_b4"]),
    ("dropped_weight_scale", "    y = y * sw;\n", "",
     ["test_golden_hand_example_b4", "test_rotation_identity_end_to_end"]),
    ("dropped_bias", "        y = y + bias[n];", "        y = y;",
     ["test_golden_hand_example_b4", "test_dequant_vs_fp64"]),
    ("bf16_tie_not_even", "(rest == 0x8000u && (keep & 1u))", "(rest == 0x8000u)",
     ["test_bf16_narrowing_matches_torch"]),
    ("gelu_wrong_arg", "erf(z / sqrt(2.0))", "erf(z * sqrt(2.0))",
     ["test_gelu_values", "test_gelu_bf16_and_mlp_chain"]),
    ("stage_stride_skip", "for (int h = 1; h < b; h *= 2)", "for (int h = 1; h < b; h *= 4)",
     ["test_fwht_columns_are_sylvester", "test_hadamard_orthogonality"]),
    ("regular_sign", "blk[i + 2 * h] = S - 2.0f * a2;", "blk[i + 2 * h] = 2.0f * a2 - S;",
     ["test_regular_columns", "test_regular_hadamard_properties"]),
    ("regular_digit_skip", "for (int h = 1; h < b; h *= 4)", "for (int h = 4; h < b; h *= 4)",
     ["test_regular_columns", "test_regular_hadamard_properties"]),
    # every exact-arithmetic pin of the Hadamard passes with the strides
    # reversed; only the hand-worked fp32 association catches it
    ("descending_strides", "for (int h = 1; h < b; h *= 2)", "for (int h = b / 2; h >= 1; h /= 2)",
     ["test_golden_fwht_stage_order"]),
    ("lowrank_bias_on_factor1", "qa, sa, r, NULL, OR_BF16, h);", "qa, sa, r, bias, OR_BF16, h);",
     ["test_lowrank_is_two_chained_linears_with_bias"]),
    ("lowrank_bias_dropped", "qb, sb, N, bias, out_dtype, out);", "qb, sb, N, NULL, out_dtype, out);",
     ["test_lowrank_is_two_chained_linears_with_bias"]),
    ("mlp_dropped_bias_up", "qu, su, F, bias_up, OR_BF16, u);", "qu, su, F, NULL, OR_BF16, u);",
     ["test_mlp_is_two_biased_linears_around_gelu"]),
    ("mlp_dropped_bias_down", "qd, sd, N, bias_down,\n                                           out_dtype, out);\n        }\n        if (rc == OR_OK && u_out)",
     "qd, sd, N, NULL,\n                                           out_dtype, out);\n        }\n        if (rc == OR_OK && u_out)",
     ["test_mlp_is_two_biased_linears_around_gelu"]),
    ("silu_sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));",
     ["test_silu_values", "test_silu_f32_every_bf16_pattern"]),
    ("swiglu_gate_up_swapped", "float sg = oracle_silu_f32(gu[m * 2 * F + j]);",
     "float sg = oracle_silu_f32(gu[m * 2 * F + F + j]);",
     ["test_swiglu_bf16_composition"]),
    ("swiglu_dropped_bias_gu", "qgu, sgu, 2 * F, bias_gu, OR_BF16, gu);",
     "qgu, sgu, 2 * F, NULL, OR_BF16, gu);",
     ["test_swiglu_mlp_is_linear_swiglu_linear"]),
    ("swiglu_down_block", "rc = oracle_linear_forward_rot(g, M, F, b_down, rot,",
     "rc = oracle_linear_forward_rot(g, M, F, b_up, rot,",
     ["test_swiglu_mlp_is_linear_swiglu_linear"]),
]

CALL = {
    "test_golden_hand_example_b4": lambda: pins.test_golden_hand_example_b4(),
    "test_rotation_identity_end_to_end": lambda: pins.test_rotation_identity_end_to_end(128, "sylvester"),
    "test_fwht_columns_are_sylvester": lambda: pins.test_fwht_columns_are_sylvester(8),
    "test_hadamard_orthogonality": lambda: pins.test_hadamard_orthogonality(64),
    "test_rowquant_rne_ties": lambda: pins.test_rowquant_rne_ties(),
    "test_rowquant_invariants": lambda: pins.test_rowquant_invariants(),
    "test_b1_is_textbook_w8a8": lambda: pins.test_b1_is_textbook_w8a8(),
    "test_gemm_brute_force_tiny": lambda: pins.test_gemm_brute_force_tiny(),
    "test_dequant_vs_fp64": lambda: pins.test_dequant_vs_fp64(),
    "test_bf16_narrowing_matches_torch": lambda: pins.test_bf16_narrowing_matches_torch(),
    "test_gelu_values": lambda: pins.test_gelu_values(),
    "test_gelu_bf16_and_mlp_chain": lambda: pins.test_gelu_bf16_and_mlp_chain(),
    "test_regular_columns": lambda: pins.test_regular_columns(64),
    "test_regular_hadamard_properties": lambda: pins.test_regular_hadamard_properties(64),
    "test_golden_fwht_stage_order": lambda: pins.test_golden_fwht_stage_order(),
    "test_lowrank_is_two_chained_linears_with_bias":
        lambda: pins.test_lowrank_is_two_chained_linears_with_bias(),
    "test_mlp_is_two_biased_linears_around_gelu":
        lambda: pins.test_mlp_is_two_biased_linears_around_gelu(),
    "test_silu_values": lambda: pins.test_silu_values(),
    "test_silu_f32_every_bf16_pattern": lambda: pins.test_silu_f32_every_bf16_pattern(),
    "test_swiglu_bf16_composition": lambda: pins.test_swiglu_bf16_composition(),
    "test_swiglu_mlp_is_linear_swiglu_linear":
        lambda: pins.test_swiglu_mlp_is_linear_swiglu_linear(),
}


@pytest.mark.parametrize("name,orig,bad,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, orig, bad, catchers):
    assert SRC.count(orig) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / f"mutant_{name}.c"
    src.write_text(SRC.replace(orig, bad))
    lib_path = tmp_path / f"libmutant_{name}.so"
    subprocess.run(["gcc", *obuild.CFLAGS, str(src), "-o", str(lib_path), "-lm"],
                   check=True, capture_output=True)
    mutant = omod.open_library(str(lib_path))
    prev = omod._swap_library(mutant)
    caught = []
    try:
        for pin in catchers:
            try:
                CALL[pin]()
            except (AssertionError, ValueError):
                caught.append(pin)
    finally:
        omod._swap_library(prev)
    assert caught, f"planted mistake {name!r} passed every pin: {catchers}"
    # the real oracle still passes the same pins
    for pin in catchers:
        CALL[pin]()
