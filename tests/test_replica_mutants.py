"""The replica pins catch plausible mistakes in the reference assignment.

Each case plants one mistake in a copy of oracle/replicas.py (loaded as a
fresh module; the real file is never modified) and runs the pin tests of
tests/test_replicas.py against it: at least one must fail. (A node count
over all choices instead of the remaining ones, or a home node taken first
even when it serves none of them, is not listed: either can pick a node that
serves nothing left and loop forever.)
"""
import os
import types

import pytest

import oracle
from tests import test_replicas as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "replicas.py")

NODE_KEY = "key=lambda n: (len(served(n)), n == hnode, -n)"
RANK_KEY = "key=lambda r: (len(held(r)), r == home, -r)"
MUTANTS = [
    ("node_ties_ignore_home", NODE_KEY, "key=lambda n: (len(served(n)), -n)"),
    ("node_ties_to_highest", NODE_KEY, "key=lambda n: (len(served(n)), n == hnode, n)"),
    ("home_node_before_count", NODE_KEY,
     "key=lambda n: (len(served(n)) > 0 and n == hnode, len(served(n)), -n)"),
    ("rank_ties_ignore_home", RANK_KEY, "key=lambda r: (len(held(r)), -r)"),
    ("rank_ties_to_highest", RANK_KEY, "key=lambda r: (len(held(r)), r == home, r)"),
    ("ranks_outside_node", "best = max(range(n * rpn, (n + 1) * rpn),",
     "best = max(range(G),"),
    ("home_rank_round_robin", "home = t * G // T", "home = t % G"),
    ("node_takes_one_choice", "for j in served(best):", "for j in served(best)[:1]:"),
    ("slots_token_major", "order = np.lexsort((j_of, t_of, e_of))", "order = np.lexsort((j_of, e_of, t_of))"),
    ("rows_token_major", "for g in range(G):\n        toks", "for g in reversed(range(G)):\n        toks"),
    ("cross_rows_count_home", "cross_rows += (g // rpn) != hnode", "cross_rows += 1"),
]


def _load(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"replicas_mutant_{name}")
    exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


def _pin_suite():
    cases = [lambda n=n: pins.test_golden_assignment(n) for n in "ABC"]
    cases += [pins.test_golden_layout, pins.test_home_rank_of_uneven_shards, pins.test_dropped_choice]
    cases += [lambda a=a: pins.test_single_copy_reduces_to_placement_layout(*a)
              for a in [(300, 32, 4, 8, 2, 0), (100, 24, 6, 6, 3, 2)]]
    cases += [lambda a=a: pins.test_everywhere_goes_home(*a) for a in [(64, 8, 2), (50, 6, 3)]]
    cases += [lambda s=s: pins.test_greedy_cover_properties(s) for s in range(2)]
    failed = 0
    for c in cases:
        try:
            c()
        except Exception:  # an assertion, or the mutant breaking outright
            failed += 1
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, monkeypatch):
    monkeypatch.setattr(pins, "rep", _load(name, old, new))
    assert _pin_suite() > 0, f"no pin caught mutant {name}"


def test_unmutated_passes_every_pin(monkeypatch):
    monkeypatch.setattr(pins, "rep", _load("none", "import numpy as np", "import numpy as np"))
    assert _pin_suite() == 0
