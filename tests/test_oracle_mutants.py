"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a private copy of oracle/moe_oracle.c, builds
it on the CPU, swaps it in, and checks that at least one pin test fails.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as P

MUTANTS = {
    "tie_break_to_higher_index": ("l[e] > l[best]", "l[e] >= l[best]"),
    "token_major_priority": ("int64_t r = q / T, t = q % T;", "int64_t t = q / k, r = q % k;"),
    "capacity_floor": ("double c = ceil(", "double c = floor("),
    "keep_one_past_capacity": ("if (!absent[i] && (C < 0 || slot[i] < C)) {", "if (!absent[i] && (C < 0 || slot[i] <= C)) {"),
    "softmax_over_selected_only": ("for (int64_t e = 0; e < E; ++e) den += exp((double)l[e] - m);",
                                   "for (int j = 0; j < k; ++j) den += exp((double)l[idx[j]] - m);"),
    "router_transposed": ("acc[e] += xv * (double)w[e];", "acc[e] += xv * (double)Wg[e * H + h];"),
    "bias_dropped": ("(float)(bias ? acc[e] + (double)bias[e] : acc[e])", "(float)(acc[e])"),
    "gelu_sign": ("0.5 * u * (1.0 + erf(", "0.5 * u * (1.0 - erf("),
    "silu_sign": ("z / (1.0 + exp(-z))", "z / (1.0 + exp(z))"),
    "down_proj_transposed": ("int64_t base = (e * H + n) * F;\n        double y = 0.0;\n        for (int64_t f = 0; f < F; ++f) y += hr[f] * elem(W2, dtype, base + f);",
                             "double y = 0.0;\n        for (int64_t f = 0; f < F; ++f) y += hr[f] * elem(W2, dtype, (e * F + f) * H + n);"),
    "combine_drops_residual": ("double acc = residual ? elem(residual, dtype, t * H + c) : 0.0;", "double acc = 0.0;"),
    "probs_keeps_smallest": ("if (x[0] != y[0]) return x[0] > y[0] ? -1 : 1;", "if (x[0] != y[0]) return x[0] < y[0] ? -1 : 1;"),
    "probs_tie_to_later": ("return x[1] < y[1] ? -1 : (x[1] > y[1] ? 1 : 0);", "return x[1] > y[1] ? -1 : (x[1] < y[1] ? 1 : 0);"),
    "sigmoid_sign": ("sc[r] = 1.0 / (1.0 + exp(-(double)l[idx[r]]));", "sc[r] = 1.0 / (1.0 + exp((double)l[idx[r]]));"),
    "sigmoid_not_renormalised": ("g[r] = (float)(mode == OR_SOFTMAX_TOPK ? sc[r] : sc[r] / sum);", "g[r] = (float)(sc[r]);"),
    "second_rule_without_2": ("absent[t * 2 + 1] = !((double)second_u[t] * (g1 + g2) < 2.0 * g2);", "absent[t * 2 + 1] = !((double)second_u[t] * (g1 + g2) < g2);"),
    "second_rule_reversed": ("absent[t * 2 + 1] = !((double)second_u[t] * (g1 + g2) < 2.0 * g2);", "absent[t * 2 + 1] = ((double)second_u[t] * (g1 + g2) < 2.0 * g2);"),
    "aux_without_k": ("f = (double)demand[e] / ((double)T * (double)k);", "f = (double)demand[e] / (double)T;"),
    "aux_without_E": ("out[0] = aux_coeff * (double)E * dot;", "out[0] = aux_coeff * dot;"),
    "zloss_not_squared": ("zsum += lse * lse;", "zsum += lse;"),
    "zloss_without_max": ("const double lse = m + log(den);", "const double lse = log(den);"),
    "renorm_missing": ("for (int r = 0; r < k; ++r) g[r] = (float)(p[r] / s);", "for (int r = 0; r < k; ++r) g[r] = (float)(p[r]);"),
}

PINS = [
    lambda: P.test_capacity_golden(),
    lambda: P.test_capacity_config_values(),
    lambda: P.test_logits_equal_correctly_rounded_exact_dot(oracle.BF16),
    lambda: P.test_selection_brute_force_all_integer_logits(3),
    lambda: P.test_selection_brute_force_all_integer_logits(4),
    lambda: P.test_two_expert_softmax_is_logistic(),
    lambda: P.test_softmax_topk_matches_library_softmax(),
    lambda: P.test_renormalised_gates_sum_to_one_and_modes_agree(),
    lambda: P.test_slot_assignment_brute_force(4, 3, 2),
    lambda: P.test_capacity_calculator_drop_scenario(),
    lambda: P.test_single_expert_is_dense_ffn(oracle.GELU, oracle.BF16),
    lambda: P.test_single_expert_is_dense_ffn(oracle.SWIGLU, oracle.BF16),
    lambda: P.test_switch_top1_output_is_gate_times_expert(),
    lambda: P.test_dropped_tokens_pass_residual_bit_exactly(),
    lambda: P.test_aux_loss_is_coefficient_for_uniform_probabilities(2, 0),
    lambda: P.test_aux_loss_hand_examples(),
    lambda: P.test_z_loss_closed_forms(),
    lambda: P.test_sigmoid_gates_closed_forms(),
    lambda: P.test_probs_policy_hand_example(),
    lambda: P.test_probs_policy_keeps_largest_gates(0),
    lambda: P.test_probs_policy_equal_gates_is_position_policy(),
    lambda: P.test_gshard_second_choice_rule(),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-w",
                    "-o", str(so), str(path), "-lm"], check=True)
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    so = _build_mutant(tmp_path, name, old, new)
    good = oracle.lib()
    mutant = ctypes.CDLL(so)
    for fn in ("oracle_capacity", "oracle_logits", "oracle_route_from_logits", "oracle_dispatch",
               "oracle_expert_rows", "oracle_expert_ffn", "oracle_combine", "oracle_token_outputs",
               "oracle_router_losses"):
        g, m = getattr(good, fn), getattr(mutant, fn)
        m.restype, m.argtypes = g.restype, g.argtypes
    caught = []
    oracle._lib = mutant
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                caught.append(pin)
    finally:
        oracle._lib = good
    assert caught, f"no pin caught mutant {name}"
