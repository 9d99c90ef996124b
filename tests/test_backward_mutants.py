"""The backward pins catch plausible mistakes in the reference.

Each case plants one mistake in a copy of oracle/backward.py (loaded as a
fresh module; the real file is never modified) and runs the pin tests of
tests/test_backward.py against it: at least one must fail.
"""
import os
import types

import pytest

import oracle
from tests import test_backward as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "backward.py")

MUTANTS = [
    ("silu_grad_is_sigmoid", "return s * (1.0 + u * (1.0 - s))", "return s"),
    ("dv_uses_silu_grad", "return dh * v * silu_grad(u), dh * silu(u)",
     "return dh * v * silu_grad(u), dh * silu_grad(u)"),
    ("dgates_no_inner", "g * (dg - inner)", "g * dg"),
    ("dgates_sign", "g * (dg - inner)", "g * (inner - dg)"),
    ("dy_without_gate", "dy[s] = g[live, j:j + 1] * dout[live]", "dy[s] = dout[live]"),
    ("da_drops_up", "da[a:b] = du[a:b] @ wg[e] + dv[a:b] @ wu[e]", "da[a:b] = du[a:b] @ wg[e]"),
    ("dw_up_from_du", "dwu[e] = dv[a:b].T @ ar[a:b]", "dwu[e] = du[a:b].T @ ar[a:b]"),
    ("dw_down_uses_u", "dwd[e] = dy[a:b].T @ h[a:b]", "dwd[e] = dy[a:b].T @ np.asarray(u, np.float64)[a:b]"),
    ("dx_first_choice_only", "dx = np.zeros((T, da.shape[1]))\n    for j in range(k):",
     "dx = np.zeros((T, da.shape[1]))\n    for j in range(1):"),
    ("dx_reads_dropped_choices", "dx[live] += da[so[live, j]]", "dx += da[so[:, j]]"),
    ("dgates_of_dropped_choice", "dgates[live, j] = (dout[live] * y[s]).sum(1)",
     "dgates[:, j] = (dout * y[so[:, j]]).sum(1)"),
    ("slot_order_token_major", "order = np.lexsort((j_of, t_of, e_of))",
     "order = np.lexsort((j_of, e_of, t_of))"),
]


def _load(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"backward_mutant_{name}")
    exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


def _pin_suite():
    cases = [lambda a=a: pins.test_gradients_match_finite_differences(*a) for a in [(0, 2)]]
    cases += [pins.test_forward_recompute_matches_c_oracle, pins.test_softmax_jacobian_invariants,
              pins.test_unused_expert_gets_zero_weight_gradient, pins.test_silu_grad_closed_forms,
              pins.test_dropped_choices_are_zero_rows]
    failed = 0
    for c in cases:
        try:
            c()
        except Exception:  # an assertion, or the mutant breaking outright
            failed += 1
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, monkeypatch):
    monkeypatch.setattr(pins, "B", _load(name, old, new))
    assert _pin_suite() > 0, f"no pin caught mutant {name}"


def test_unmutated_passes_every_pin(monkeypatch):
    monkeypatch.setattr(pins, "B", _load("none", "import numpy as np", "import numpy as np"))
    assert _pin_suite() == 0
