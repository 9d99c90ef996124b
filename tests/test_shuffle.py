"""Pins of the reference token shuffling and locality statistic
(oracle/shuffle.py).

Source: Zyphra correlated expert placement page, English abstract (token
shuffling; the page reports the on-GPU share 12.5% -> 59% on one node). The
reading: a token should sit where most of its next-layer experts are served,
which beats the 1/G share of uniform routing (12.5% on 8 GPUs). Pinned by

* the hand-worked examples in tests/golden/token_shuffle_worked_example.txt
  (both tie rules, the lowest-rank fallback, a one-hot and a general
  affinity table, indices that are not experts, the shuffled order and the
  served counts);
* the closed form: under uniform routing and a balanced placement the home
  share has mean 1/G (checked within 4 standard deviations of the
  hypergeometric count);
* brute-force properties: the destination maximises the summed affinity (a
  vectorised recount with numpy gathers); with a one-hot placement table it
  holds the most of the token's experts, so serving there never loses to
  serving at home; a batch already at home does not move; the shuffled order
  is a stable sort with the inverse permutation and per-rank offsets.
"""
import os

import numpy as np
import pytest

from oracle import shuffle as sh

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_shuffle_worked_example.txt")


def load_golden():
    cases, cur = {}, None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("case "):
            cur = cases.setdefault(line.split()[1], {})
            continue
        key, val = line.split(":", 1)
        cur[key] = [int(v) for v in val.split()]
    for c in cases.values():
        for key in ("G", "E", "k", "served_home", "served_dest"):
            if key in c:
                c[key] = c[key][0]
        c["want"] = np.array(c["want"], np.int32).reshape(-1, c["k"])
    return cases


@pytest.mark.parametrize("name", ["A", "B"])
def test_golden(name):
    c = load_golden()[name]
    aff = (np.array(c["aff"]).reshape(c["E"], c["G"]) if "aff" in c
           else sh.onehot(c["place"], c["G"]))
    dest = sh.destinations(c["want"], aff, c["G"])
    assert dest.tolist() == c["dest"]
    s = sh.shuffle(dest, c["G"])
    for key in ("perm", "rank_off", "pos"):
        assert s[key].tolist() == c[key], key
    if "served_home" in c:
        T, k = c["want"].shape
        home = sh.home_ranks(T, c["G"])
        assert sh.local_share(c["want"], c["place"], home) * T * k == pytest.approx(c["served_home"])
        assert sh.local_share(c["want"], c["place"], dest) * T * k == pytest.approx(c["served_dest"])


def _uniform_topk(T, E, k, seed):
    rng = np.random.default_rng(seed)
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("E,k,G", [(64, 4, 8), (128, 8, 16), (32, 2, 4)])
def test_uniform_home_share_is_one_over_G(E, k, G):
    T = 20000
    idx = _uniform_topk(T, E, k, E + k)
    place = np.repeat(np.arange(G), E // G).astype(np.int32)
    share = sh.local_share(idx, place, sh.home_ranks(T, G))
    p = 1.0 / G
    var_count = k * p * (1 - p) * (E - k) / (E - 1)   # hypergeometric count per token
    sd = np.sqrt(var_count / T) / k
    assert abs(share - p) < 4 * sd


def _counts(want, place, G):
    ranks = np.asarray(place)[want]
    return np.stack([(ranks == g).sum(1) for g in range(G)], axis=1)   # [T, G]


@pytest.mark.parametrize("seed", range(3))
def test_destination_holds_most_and_beats_home(seed):
    T, E, k, G = 400, 32, 6, 8
    rng = np.random.default_rng(seed)
    place = rng.integers(0, G, size=E).astype(np.int32)
    want = _uniform_topk(T, E, k, seed + 5)
    dest = sh.destinations(want, sh.onehot(place, G), G)
    cnt = _counts(want, place, G)
    home = sh.home_ranks(T, G)
    assert (cnt[np.arange(T), dest] == cnt.max(1)).all()
    best = cnt == cnt.max(1, keepdims=True)
    home_best = best[np.arange(T), home]
    assert (dest[home_best] == home[home_best]).all()
    first = best.argmax(1)
    assert (dest[~home_best] == first[~home_best]).all()
    assert sh.local_share(want, place, dest) >= sh.local_share(want, place, home)


def test_batch_at_home_does_not_move():
    T, G, k = 64, 8, 3
    place = np.repeat(np.arange(G), 4).astype(np.int32)
    home = sh.home_ranks(T, G)
    want = np.stack([home * 4 + j for j in range(k)], axis=1).astype(np.int32)
    dest = sh.destinations(want, sh.onehot(place, G), G)
    assert (dest == home).all()
    s = sh.shuffle(dest, G)
    assert s["perm"].tolist() == list(range(T))
    assert sh.local_share(want, place, dest) == 1.0


@pytest.mark.parametrize("seed", range(3))
def test_destination_maximises_affinity(seed):
    T, E, k, G = 300, 16, 4, 6
    rng = np.random.default_rng(seed)
    aff = rng.integers(0, 4, size=(E, G))
    want = _uniform_topk(T, E, k, seed + 4)
    want[rng.random((T, k)) < 0.1] = -1          # not an expert: adds nothing
    dest = sh.destinations(want, aff, G)
    valid = want >= 0
    score = (aff[np.where(valid, want, 0)] * valid[:, :, None]).sum(1)   # [T, G]
    best = score == score.max(1, keepdims=True)
    home = sh.home_ranks(T, G)
    want_dest = np.where(best[np.arange(T), home], home, best.argmax(1))
    assert np.array_equal(dest, want_dest)


def test_onehot_table():
    assert sh.onehot([2, 0, 2], 3).tolist() == [[0, 0, 1], [1, 0, 0], [0, 0, 1]]


@pytest.mark.parametrize("seed", range(3))
def test_shuffle_is_stable_sort(seed):
    rng = np.random.default_rng(seed)
    T, G = 500, 7
    dest = rng.integers(0, G, size=T).astype(np.int32)
    s = sh.shuffle(dest, G)
    perm, pos, off = s["perm"], s["pos"], s["rank_off"]
    assert sorted(perm.tolist()) == list(range(T))
    d = dest[perm]
    assert (np.diff(d) >= 0).all()
    same = np.diff(d) == 0
    assert (np.diff(perm)[same] > 0).all()
    assert (pos[perm] == np.arange(T)).all()
    for g in range(G):
        assert (d[off[g]:off[g + 1]] == g).all()
    assert off[-1] == T


def test_no_prediction_stays_home_on_uneven_shards():
    T, G = 10, 4
    want = np.full((T, 2), -1, np.int32)
    dest = sh.destinations(want, np.ones((4, G), np.int64), G)
    assert dest.tolist() == [0, 0, 0, 1, 1, 2, 2, 2, 3, 3]


def test_offsets_with_empty_ranks():
    s = sh.shuffle(np.array([1, 1, 0, 1], np.int32), 4)
    assert s["rank_off"].tolist() == [0, 1, 4, 4, 4]
    assert s["perm"].tolist() == [2, 0, 1, 3]
