"""The placement pins catch plausible mistakes in the reference planner.

Each case plants one mistake in a copy of oracle/placement.py (loaded as a
fresh module; the real file is never modified) and runs the pin tests of
tests/test_placement.py against it: at least one must fail. (A stage 2 that
also accepts swaps leaving the larger load unchanged is not listed: it can
swap back and forth forever, e.g. on loads 4 1 2 1 with E=4, G=2.)
"""
import importlib.util
import os
import types

import pytest

import oracle
from tests import test_placement as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "placement.py")

MUTANTS = [
    ("seed_lightest", "seed = max(free, key=lambda e: (load[e], -e))",
     "seed = min(free, key=lambda e: (load[e], e))"),
    ("growth_ignores_weights", "u = max(free, key=lambda e: (int(w[e, members].sum()), load[e], -e))",
     "u = max(free, key=lambda e: (load[e], -e))"),
    ("growth_ties_to_higher_index", "u = max(free, key=lambda e: (int(w[e, members].sum()), load[e], -e))",
     "u = max(free, key=lambda e: (int(w[e, members].sum()), load[e], e))"),
    ("swap_accepts_ties", "swap_delta(w, place, a, b) > 0", "swap_delta(w, place, a, b) >= 0"),
    ("no_swap_refinement", "for _ in range(swap_passes):", "for _ in range(0):"),
    ("one_sided_weights", "w = c + c.T", "w = c.copy()"),
    ("stage2_neighbour_not_lightest", "l = min(ranks, key=lambda r: (L[r], r))",
     "l = ranks[(ranks.index(h) + 1) % len(ranks)]"),
    ("stage2_worst_swap", "key = (nm, -swap_delta(w, place, a, b), a, b)",
     "key = (-nm, -swap_delta(w, place, a, b), a, b)"),
    ("stage2_crosses_nodes", "ranks = list(range(n0, n0 + rpn))", "ranks = list(range(0, G))"),
    ("rows_count_slots", "(np.diff(ranks, axis=1) != 0).sum()", "(np.diff(ranks, axis=1) >= 0).sum()"),
]


def _load(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"placement_mutant_{name}")
    exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


def _pin_suite():
    cases = [pins.test_golden_worked_example, pins.test_dispatched_rows_definition]
    cases += [lambda n=n: pins.test_zero_input_is_contiguous(n) for n in (0, 1, 3, 8)]
    cases += [lambda a=a: pins.test_planted_clusters_recovered(*a) for a in [(16, 4, 0), (32, 4, 1)]]
    cases += [lambda a=a: pins.test_planted_clusters_recovered_by_growth_alone(*a)
              for a in [(16, 4, 10), (32, 8, 11)]]
    cases += [lambda a=a: pins.test_balanced_ranks(*a) for a in [(24, 6, 1, 3), (32, 8, 4, 4)]]
    cases += [lambda s=s: pins.test_stage1_is_swap_local_optimum(s) for s in range(2)]
    cases += [lambda s=s: pins.test_brute_force_optimum_e4_g2(s) for s in range(6)]
    cases += [lambda s=s: pins.test_stage2_rebalances_within_nodes(s) for s in range(3)]
    failed = 0
    for c in cases:
        try:
            c()
        except Exception:  # an assertion, or the mutant breaking outright
            failed += 1
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, monkeypatch):
    monkeypatch.setattr(pins, "P", _load(name, old, new))
    assert _pin_suite() > 0, f"no pin caught mutant {name}"


def test_unmutated_passes_every_pin(monkeypatch):
    monkeypatch.setattr(pins, "P", _load("none", "import numpy as np", "import numpy as np"))
    assert _pin_suite() == 0
