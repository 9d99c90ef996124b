"""The pins catch plausible mistakes in the reference.

Each case plants one mistake in a copy of oracle.c (on the CPU), builds it,
and runs a selection of the pin tests against that build: at least one pin
must fail. The real oracle.c is never modified.
"""
import os

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = [
    ("tie_to_higher_index", "return la > lb || (la == lb && ia < ib);",
     "return la > lb || (la == lb && ia > ib);"),
    ("group_score_min", "if ((double)l[e] > s) s = (double)l[e];",
     "if ((double)l[e] < s) s = (double)l[e];"),
    ("gate_denominator_drops_term",
     "for (int j = 0; j < k; ++j) den += exp(", "for (int j = 1; j < k; ++j) den += exp("),
    ("gate_numerator_wrong_slot",
     "gates[(size_t)t * k + j] = exp((double)l[topk_idx[(size_t)t * k + j]] - l0) / den;",
     "gates[(size_t)t * k + j] = exp((double)l[topk_idx[(size_t)t * k]] - l0) / den;"),
    ("coact_counts_diagonal", "if (i == j) continue;", "(void)0;"),
    ("coact_one_order_only", "if (i == j) continue;", "if (i >= j) continue;"),
    ("row_of_wrong_rank", "perm_row[s] = row_of[(size_t)t * G + place[e]];",
     "perm_row[s] = row_of[(size_t)t * G + place[topk_idx[(size_t)t * k]]];"),
    ("rank_mask_drops_last_slot",
     "for (int j = 0; j < k; ++j) m |= 1u << place[",
     "for (int j = 0; j + 1 < k; ++j) m |= 1u << place["),
    ("silu_sign", "h[f] = u / (1.0 + exp(-u)) * v;", "h[f] = u / (1.0 + exp(u)) * v;"),
    ("gate_up_swapped", "h[f] = u / (1.0 + exp(-u)) * v;", "h[f] = v / (1.0 + exp(-v)) * u;"),
    ("no_silu", "h[f] = u / (1.0 + exp(-u)) * v;", "h[f] = u * v;"),
    ("down_transposed", "size_t wo = (e * (size_t)d + (size_t)n) * (size_t)F;\n            double acc = 0.0;\n            for (int f = 0; f < F; ++f) acc += orc_elem(w_down, wo + (size_t)f, dt) * h[f];",
     "size_t wo = e * (size_t)d * (size_t)F + (size_t)n;\n            double acc = 0.0;\n            for (int f = 0; f < F; ++f) acc += orc_elem(w_down, wo + (size_t)f * (size_t)d, dt) * h[f];"),
    ("up_uses_gate_weights", "v += orc_elem(w_up, wo + (size_t)c, dt) * a[c];",
     "v += orc_elem(w_gate, wo + (size_t)c, dt) * a[c];"),
    ("combine_ignores_gate", "acc += gates[(size_t)t * k + j] * y[", "acc += 1.0 * y["),
    ("combine_first_gate_only", "acc += gates[(size_t)t * k + j] * y[", "acc += gates[(size_t)t * k] * y["),
    ("bf16_widen_wrong_shift", "<< 16;\n    float f;", "<< 15;\n    float f;"),
    ("combine_dropped_reads_slot0", "if (s < 0) continue;", "if (s < 0) s = 0;"),
]


def _pin_suite(orc):
    """Run a fast selection of pins; return the number that failed."""
    cases = []
    cases += [lambda s=s: pins.test_route_brute_force_with_ties(orc, s) for s in range(12)]
    cases += [lambda s=s: pins.test_route_group_limited_brute_force(orc, s) for s in range(10)]
    cases += [lambda: pins.test_route_k1_gate_is_one_and_two_way_logistic(orc),
              lambda: pins.test_route_vs_lexsort_on_workloads(orc, 0),
              lambda: pins.test_coact_tiny_brute(orc),
              lambda: pins.test_coact_closed_form_and_invariants(orc, 0)]
    cases += [lambda s=s: pins.test_layout_small_random(orc, s) for s in range(6)]
    cases += [lambda: pins.test_layout_on_workloads(orc, 0, "contiguous"),
              lambda: pins.test_ffn_vs_matmul(orc, "f32"),
              lambda: pins.test_ffn_vs_matmul(orc, "bf16"),
              lambda: pins.test_combine_k1_is_permutation(orc),
              lambda: pins.test_combine_dropped_choice_is_a_zero_term(orc),
              lambda: pins.test_layer_k_equals_E_is_dense_mixture(orc),
              lambda: pins.test_layer_vs_numpy_pipeline(orc, "f32")]
    failed = 0
    for c in cases:
        try:
            c()
        except (AssertionError, ValueError):
            failed += 1
    return failed


def test_unmutated_copy_passes(tmp_path):
    src = open(oracle._SRC).read()
    p = tmp_path / "o.c"
    p.write_text(src)
    lib = oracle.compile_c(str(p), str(tmp_path / "lib.so"))
    with oracle.use_library(lib):
        assert _pin_suite(oracle) == 0


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(oracle._SRC).read()
    assert old in src, f"mutation anchor for {name} not found"
    p = tmp_path / "o.c"
    p.write_text(src.replace(old, new, 1))
    lib = oracle.compile_c(str(p), str(tmp_path / "lib.so"))
    with oracle.use_library(lib):
        assert _pin_suite(oracle) > 0, f"no pin caught mutant {name}"
