"""The backward pins must catch plausible mistakes in the backward oracle.

Each case plants one mistake in a private copy of oracle/backward.py, loads it as a
module, points the pin tests at it, and checks that at least one pin fails.
"""
import importlib.util
import os
import sys

import pytest

from tests import test_oracle_backward_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "backward.py")

MUTANTS = {
    "softmax_topk_without_projection": ("        dl -= p * (g * dg).sum(1, keepdims=True)\n", ""),
    "silu_derivative_is_silu": ("    return s * (1.0 + a * (1.0 - s))", "    return s"),
    "gelu_derivative_without_density": (
        "0.5 * (1.0 + erf(u / SQRT2)) + u * np.exp(-0.5 * u * u) / np.sqrt(2.0 * np.pi)",
        "0.5 * (1.0 + erf(u / SQRT2))"),
    "down_grad_uses_preactivation": ("        dW2[e] = dYe.T @ z", "        dW2[e] = dYe.T @ u"),
    "input_grad_without_up_branch": ("            dX[lo:hi] = du @ W1[e] + dv @ W3[e]", "            dX[lo:hi] = du @ W1[e]"),
    "up_grad_without_gate": ("            dv = dz * _silu(u)", "            dv = dz"),
    "gate_grad_on_dropped_choices": ("        kept = np.nonzero(dst[:, r] >= 0)[0]\n        rows = dst[kept, r]",
                                     "        kept = np.arange(T)\n        rows = dst[kept, r]"),
    "output_grad_without_gate": ("        dY[rows] = g[kept, r][:, None] * dy[kept]", "        dY[rows] = dy[kept]"),
    "renorm_as_softmax_over_all": ("    if gate_mode == SOFTMAX_TOPK:\n        p = _softmax(l)",
                                   "    if gate_mode != TOPK_SOFTMAX:\n        p = _softmax(l)"),
    "sigmoid_without_derivative": ("        np.add.at(dl, (np.broadcast_to(tt, idx.shape), idx), dsc * ds_dl)",
                                   "        np.add.at(dl, (np.broadcast_to(tt, idx.shape), idx), dsc)"),
    "aux_sign": ("            dl += p * (c[None, :] - (p * c[None, :]).sum(1, keepdims=True))",
                 "            dl -= p * (c[None, :] - (p * c[None, :]).sum(1, keepdims=True))"),
    "zloss_without_factor_two": ("        dl += z_coeff * 2.0 / T * lse[:, None] * _softmax(l)",
                                 "        dl += z_coeff / T * lse[:, None] * _softmax(l)"),
    "dispatch_grad_overwrites": ("        dx[kept] += dX[dst[kept, r]]", "        dx[kept] = dX[dst[kept, r]]"),
    "bias_grad_row_sum": ("    return dl @ W.T, xf.T @ dl, dl.sum(0)", "    return dl @ W.T, xf.T @ dl, dl.sum(0) * 0.5"),
}

PINS = [
    *[(lambda c=c: P.test_layer_gradient_matches_finite_differences(c)) for c in range(len(P.CASES))],
    lambda: P.test_softmax_gate_gradients_sum_to_zero_per_token(),
    lambda: P.test_single_expert_has_no_router_gradient(),
    lambda: P.test_bias_gradient_is_column_sum_and_router_transpose(),
    lambda: P.test_combine_and_dispatch_backward_are_the_all_to_all_transposes(),
]


def _load_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path = tmp_path / f"backward_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"oracle._mutant_{name}", str(path))
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    mutant = _load_mutant(tmp_path, name, old, new)
    good = P.OB
    caught = []
    P.OB = mutant
    try:
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                caught.append(pin)
    finally:
        P.OB = good
    assert caught, f"no pin caught mutant {name}"
