"""The oracle's pins must reject plausible mistakes.

Each case below plants one mistake in a private copy of the oracle's C
source (on the CPU, in a temporary directory), builds it, points the oracle
module at the broken build, and runs the fast pins.  At least one pin has
to fail for every mutant; the real build is restored afterwards.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins
import test_oracle_pins_ex as pins_ex
import test_oracle_pins_bf16m as pins_m
import test_oracle_pins_kahan as pins_k

MUTANTS = {
    "drop_last_rank": ("for (int k = 1; k < n_ranks; ++k)", "for (int k = 1; k < n_ranks - 1; ++k)"),
    "divide_by_n_minus_1": ("(float)(s / (double)n_ranks)", "(float)(s / (double)(n_ranks > 1 ? n_ranks - 1 : 1))"),
    "sum_not_mean": ("(float)(s / (double)n_ranks)", "(float)s"),
    "wrong_partial_index": ("return bf16_value(((const uint16_t *)p)[i]);",
                            "return bf16_value(((const uint16_t *)p)[i ^ 1]);"),
    "m_weight_swapped": ("hp->beta1 * (double)*m + (1.0 - hp->beta1) * g",
                         "(1.0 - hp->beta1) * (double)*m + hp->beta1 * g"),
    "v_uses_beta1": ("hp->beta2 * (double)*v + (1.0 - hp->beta2) * (g * g)",
                     "hp->beta1 * (double)*v + (1.0 - hp->beta1) * (g * g)"),
    "v_not_squared": ("(1.0 - hp->beta2) * (g * g)", "(1.0 - hp->beta2) * fabs(g)"),
    "no_bias_correction": ("double mhat = m1 / bc1;", "double mhat = m1;"),
    "no_v_bias_correction": ("double vhat = v1 / bc2;", "double vhat = v1;"),
    "eps_inside_sqrt": ("sqrt(vhat) + hp->eps", "sqrt(vhat + hp->eps)"),
    "decay_not_scaled_by_lr": ("(1.0 - hp->lr * hp->weight_decay)", "(1.0 - hp->weight_decay)"),
    "decay_dropped": ("(1.0 - hp->lr * hp->weight_decay)", "1.0"),
    "update_sign": ("- hp->lr * upd", "+ hp->lr * upd"),
    "step_off_by_one": ("pow(beta, (double)t)", "pow(beta, (double)(t - 1))"),
    "stale_m_used": ("double mhat = m1 / bc1;", "double mhat = (double)*m / bc1;"),
    "bf16_ties_away": ("(dropped == 0x8000u && (hi & 1u))", "(dropped == 0x8000u)"),
    "bf16_truncate": ("hi = (uint16_t)(hi + 1u);", "hi = hi;"),
    "shard_len_floor": ("int64_t S = (total + n_ranks - 1) / n_ranks;", "int64_t S = total / n_ranks;"),
    "segment_offset": ("seg[4 * count + 1] = x - a;", "seg[4 * count + 1] = x - lo;"),
    "group_transposed": ("t = t + partial_at(partials[m * group + k], gdt, i);",
                         "t = t + partial_at(partials[k * (n_ranks / group) + m], gdt, i);"),
    "group_head_transposed": ("double t = partial_at(partials[m * group], gdt, i);",
                              "double t = partial_at(partials[m], gdt, i);"),
    "grouped_flat_fold": ("        s = (m == 0) ? t : s + t;\n", "        s = s + t;\n"),
    "acc_ignored": ("        s = (double)acc[i] + s;\n", "        s = s;\n"),
    "divisor_ignores_micro_batches": ("(double)n_ranks * (double)micro_batches", "(double)n_ranks"),
    "accumulate_reset_ignored": ("acc[i] = reset ? (float)s : (float)((double)acc[i] + s);",
                                 "acc[i] = (float)((double)acc[i] + s);"),
    "bf16d_truncates": ("r = ldexp(rint(ldexp(a, -q)), q);", "r = ldexp(floor(ldexp(a, -q)), q);"),
    "bf16d_spacing": ("int q = E - 8;", "int q = E - 9;"),
    "bf16m_moment_through_fp32": ("m[i] = oracle_bf16_from_double(m1);",
                                  "m[i] = oracle_bf16_round((float)m1);"),
    "bf16m_v_from_m": ("v[i] = oracle_bf16_from_double(v1);", "v[i] = oracle_bf16_from_double(m1);"),
    "bf16m_beta_swapped": ("hp->beta1 * bf16_value(m[i]) + (1.0 - hp->beta1) * g",
                           "(1.0 - hp->beta1) * bf16_value(m[i]) + hp->beta1 * g"),
    "kahan_comp_ignored": ("double y = d + bf16_value(*comp);", "double y = d;"),
    "kahan_comp_sign": ("double y = d + bf16_value(*comp);", "double y = d - bf16_value(*comp);"),
    "kahan_residual_sign": ("*comp = oracle_bf16_from_double(y - moved);",
                            "*comp = oracle_bf16_from_double(moved - y);"),
    "kahan_comp_reset": ("*comp = oracle_bf16_from_double(y - moved);", "*comp = 0;"),
    "kahan_theta_via_fp32": ("uint16_t t1 = oracle_bf16_from_double(th + y);",
                             "uint16_t t1 = oracle_bf16_round((float)(th + y));"),
    "kahan_decay_dropped": ("(upd + hp->weight_decay * bf16_value(theta[i]))", "(upd)"),
    "kahan_decay_unscaled": ("-hp->lr * (upd + hp->weight_decay * bf16_value(theta[i]))",
                             "-(hp->lr * upd + hp->weight_decay * bf16_value(theta[i]))"),
    "kahan_update_sign": ("double d = -hp->lr * (upd", "double d = hp->lr * (upd"),
    "kahan_moment_from_theta": ("double m1 = hp->beta1 * bf16_value(m[i]) + (1.0 - hp->beta1) * g;\n        double v1 = hp->beta2 * bf16_value(v[i]) + (1.0 - hp->beta2) * (g * g);\n        double mhat = m1 / bc1;\n        double vhat = v1 / bc2;\n        double upd = mhat / (sqrt(vhat) + hp->eps);\n        double d",
                                "double m1 = hp->beta1 * bf16_value(m[i]) + (1.0 - hp->beta1) * g;\n        double v1 = hp->beta2 * bf16_value(m[i]) + (1.0 - hp->beta2) * (g * g);\n        double mhat = m1 / bc1;\n        double vhat = v1 / bc2;\n        double upd = mhat / (sqrt(vhat) + hp->eps);\n        double d"),
    "accumulate_rounds_twice": ("acc[i] = reset ? (float)s : (float)((double)acc[i] + s);",
                                "acc[i] = reset ? (float)s : (float)((double)acc[i] + (double)(float)s);"),
}

FAST_PINS = [
    lambda: pins.test_bf16_round_special_values(),
    lambda: pins.test_reduce_equals_exact_rational_mean(3),
    lambda: pins.test_reduce_equals_exact_rational_mean(8),
    lambda: pins.test_gradient_averaging_identity_linear_model("f32"),
    lambda: pins.test_allreduce_equals_reduce_scatter_plus_all_gather(),
    lambda: pins.test_adamw_matches_torch_adamw_float64(pins.HP_VARIANTS[0]),
    lambda: pins.test_adamw_step1_closed_form(),
    lambda: pins.test_adamw_zero_gradient_decay_only(),
    lambda: pins.test_adamw_zero_betas_reduce_to_normalised_step(),
    lambda: pins.test_adamw_constant_gradient_unbiased_moments(),
    lambda: [pins.test_shard_segments_brute_force(s) for s in range(6)],
    lambda: pins_ex.test_one_group_and_singleton_groups_are_the_flat_order(8),
    lambda: pins_ex.test_grouping_decides_the_rounding(),
    lambda: pins_ex.test_grouped_mean_is_exact_when_sums_are_exact(8, 2),
    lambda: pins_ex.test_accumulated_micro_batches_give_the_full_batch_gradient(2),
    lambda: pins_ex.test_accumulator_rounds_once_per_micro_batch(),
    lambda: pins_m.test_double_to_bf16_matches_brute_force(),
    lambda: pins_m.test_double_to_bf16_is_one_rounding(),
    lambda: pins_m.test_bf16_moment_step_equals_fp32_step_when_moments_are_exact(),
    lambda: pins_m.test_bf16_moment_step_rounds_moments_to_nearest(),
    lambda: pins_m.test_bf16_moment_step_rounds_once(),
    lambda: pins_k.test_compensation_recovers_increments_a_bf16_sum_drops(),
    lambda: pins_k.test_no_increment_is_lost_while_the_residual_fits(0, K=60),
    lambda: pins_k.test_each_stored_value_is_the_nearest_bf16(n=400),
    lambda: pins_k.test_pure_decay_is_followed_where_plain_bf16_stalls(),
    lambda: pins_k.test_first_step_closed_form(n=400),
    lambda: pins_k.test_moments_are_those_of_the_bf16_moment_step(),
]


def _failing_pins():
    failed = 0
    for pin in FAST_PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    return failed


def test_real_oracle_passes_fast_pins():
    assert _failing_pins() == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mutant.c")
        so = os.path.join(d, "libmutant.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
                        "-shared", "-w", "-o", so, c, "-lm"], check=True)
        oracle.use_library(so)
        try:
            failed = _failing_pins()
        finally:
            oracle.use_library(None)
    assert failed >= 1, f"no pin caught mutant {name}"
