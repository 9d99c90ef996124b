"""The shuffle pins catch plausible mistakes in the reference.

Each case plants one mistake in a copy of oracle/shuffle.py (loaded as a
fresh module; the real file is never modified) and runs the pin tests of
tests/test_shuffle.py against it: at least one must fail.
"""
import os
import types

import pytest

import oracle
from tests import test_shuffle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "shuffle.py")

KEY = "key=lambda r: (score[r], r == home, -r)"
MUTANTS = [
    ("ties_ignore_home", KEY, "key=lambda r: (score[r], -r)"),
    ("ties_to_highest", KEY, "key=lambda r: (score[r], r == home, r)"),
    ("home_before_score", KEY, "key=lambda r: (r == home, score[r], -r)"),
    ("home_round_robin", "home = t * G // T", "home = t % G"),
    ("score_counts_experts", "score[g] += int(aff[e, g])", "score[g] += int(aff[e, g] > 0)"),
    ("last_expert_dropped", "if 0 <= e < E:\n", "if 0 <= e < E - 1:\n"),
    ("onehot_transposed", "aff[np.arange(len(place)), place] = 1", "aff[place, np.arange(len(place)) % G] = 1"),
    ("unstable_order", 'perm = np.argsort(dest, kind="stable").astype(np.int32)',
     'perm = (len(dest) - 1 - np.argsort(dest[::-1], kind="stable"))[::-1].astype(np.int32)'),
    ("offsets_drop_empty_ranks", "np.bincount(dest, minlength=G)", "np.bincount(dest)"),
    ("share_counts_other_ranks", "return float((ranks == np.asarray(token_rank)[:, None]).mean())",
     "return float((ranks != np.asarray(token_rank)[:, None]).mean())"),
]


def _load(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"shuffle_mutant_{name}")
    exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


def _pin_suite():
    cases = [lambda n=n: pins.test_golden(n) for n in "AB"]
    cases += [lambda a=a: pins.test_uniform_home_share_is_one_over_G(*a) for a in [(64, 4, 8)]]
    cases += [lambda s=s: pins.test_destination_holds_most_and_beats_home(s) for s in range(2)]
    cases += [lambda s=s: pins.test_destination_maximises_affinity(s) for s in range(2)]
    cases += [pins.test_batch_at_home_does_not_move, pins.test_onehot_table,
              pins.test_no_prediction_stays_home_on_uneven_shards, pins.test_offsets_with_empty_ranks]
    cases += [lambda s=s: pins.test_shuffle_is_stable_sort(s) for s in range(2)]
    failed = 0
    for c in cases:
        try:
            c()
        except Exception:  # an assertion, or the mutant breaking outright
            failed += 1
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, monkeypatch):
    monkeypatch.setattr(pins, "sh", _load(name, old, new))
    assert _pin_suite() > 0, f"no pin caught mutant {name}"


def test_unmutated_passes_every_pin(monkeypatch):
    monkeypatch.setattr(pins, "sh", _load("none", "import numpy as np", "import numpy as np"))
    assert _pin_suite() == 0
