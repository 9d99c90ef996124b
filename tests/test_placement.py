"""Expert placement planner: the oracle against its pins, then the native
planner (host code in libmoe, no GPU) against the oracle, bit for bit.

Pins: the hand-worked example in tests/golden/placement_worked_example.txt;
exact recovery of planted co-activation clusters; E/G experts per rank;
stage 1 leaves no improving pairwise swap (checked with a separately written
loop count of the within-rank weight); the brute-force optimum for E=4, G=2
(where every balanced partition is one swap from any other); the all-zero
input, which reduces to the contiguous placement; stage 2 keeps each node's
experts, never raises a node's largest rank load and leaves no improving
swap between a node's most and least loaded ranks.
"""
import itertools
import os

import numpy as np
import pytest

from oracle import placement as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "placement_worked_example.txt")


def loop_weight(coact, place):
    """Within-rank weight, written out with plain loops."""
    E = len(place)
    tot = 0
    for a in range(E):
        for b in range(a + 1, E):
            if place[a] == place[b]:
                tot += int(coact[a][b]) + int(coact[b][a])
    return tot


def planted(E, G, seed, strong=100, noise=20):
    rng = np.random.default_rng(seed)
    clusters = rng.permutation(E).reshape(G, E // G)
    c = np.zeros((E, E), np.int64)
    for grp in clusters:
        for a in grp:
            for b in grp:
                if a != b:
                    c[a, b] = strong + rng.integers(0, 10)
    n = rng.integers(0, noise, (E, E))
    c += n + n.T
    np.fill_diagonal(c, 0)
    load = rng.integers(10, 100, E)
    return c, load, clusters


def partition(place):
    return sorted(sorted(np.flatnonzero(place == g).tolist()) for g in np.unique(place))


def test_golden_worked_example():
    vals = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            vals[k] = [int(x) for x in v]
    E, G, rpn = vals["E"][0], vals["G"][0], vals["ranks_per_node"][0]
    got = P.plan(np.zeros((E, E), np.int64), vals["load"], G, rpn)
    assert got.tolist() == vals["place"]


@pytest.mark.parametrize("E,G,seed", [(16, 4, 0), (32, 4, 1), (64, 8, 2)])
def test_planted_clusters_recovered(E, G, seed):
    c, load, clusters = planted(E, G, seed)
    got = P.plan(c, load, G)
    assert partition(got) == sorted(sorted(x.tolist()) for x in clusters)


@pytest.mark.parametrize("E,G,seed", [(16, 4, 10), (32, 8, 11)])
def test_planted_clusters_recovered_by_growth_alone(E, G, seed):
    """With strong clusters the greedy fill alone (no swap passes) finds
    them: a seed's cluster mates carry the largest weights."""
    c, load, clusters = planted(E, G, seed, strong=1000, noise=5)
    got = P.plan(c, load, G, 1, swap_passes=0)
    assert partition(got) == sorted(sorted(x.tolist()) for x in clusters)


@pytest.mark.parametrize("E,G,rpn,seed", [(24, 6, 1, 3), (32, 8, 4, 4), (12, 12, 4, 5), (8, 1, 1, 6)])
def test_balanced_ranks(E, G, rpn, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 50, (E, E))
    got = P.plan(c, rng.integers(0, 100, E), G, rpn)
    assert np.array_equal(np.bincount(got, minlength=G), np.full(G, E // G))


@pytest.mark.parametrize("seed", range(4))
def test_stage1_is_swap_local_optimum(seed):
    rng = np.random.default_rng(100 + seed)
    E, G = 12, 3
    c = rng.integers(0, 30, (E, E))
    place = P.plan(c, rng.integers(0, 50, E), G, 1, swap_passes=50)
    base = loop_weight(c, place)
    for a, b in itertools.combinations(range(E), 2):
        if place[a] != place[b]:
            q = place.copy()
            q[a], q[b] = q[b], q[a]
            assert loop_weight(c, q) <= base


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_optimum_e4_g2(seed):
    rng = np.random.default_rng(200 + seed)
    c = rng.integers(0, 40, (4, 4))
    best = max(loop_weight(c, np.array(p)) for p in ([0, 0, 1, 1], [0, 1, 0, 1], [0, 1, 1, 0]))
    assert loop_weight(c, P.plan(c, rng.integers(0, 9, 4), 2)) == best


@pytest.mark.parametrize("passes", [0, 1, 3, 8])
def test_zero_input_is_contiguous(passes):
    """No weights and equal loads: the greedy fill takes experts in index
    order, and no swap raises W, so any number of passes keeps it."""
    E, G = 16, 4
    got = P.plan(np.zeros((E, E), np.int64), np.ones(E, np.int64), G, 1, passes)
    assert got.tolist() == [e // (E // G) for e in range(E)]


@pytest.mark.parametrize("seed", range(3))
def test_stage2_rebalances_within_nodes(seed):
    rng = np.random.default_rng(300 + seed)
    E, G, rpn = 32, 8, 4
    c = rng.integers(0, 30, (E, E))
    load = rng.integers(0, 200, E)
    s1 = P.plan(c, load, G, 1)
    s2 = P.plan(c, load, G, rpn)
    for n0 in range(0, G, rpn):
        node1 = np.isin(s1, range(n0, n0 + rpn))
        node2 = np.isin(s2, range(n0, n0 + rpn))
        assert np.array_equal(node1, node2)               # experts stay in their node
        L1 = P.rank_loads(load, s1, G)[n0:n0 + rpn]
        L2 = P.rank_loads(load, s2, G)[n0:n0 + rpn]
        assert L2.max() <= L1.max() and L2.sum() == L1.sum()
        h = n0 + int(np.argmax(L2)); l = n0 + int(np.argmin(L2))
        for a in np.flatnonzero(s2 == h):
            for b in np.flatnonzero(s2 == l):
                d = int(load[a] - load[b])
                if d > 0:
                    assert max(L2.max() - d, L2.min() + d) >= L2.max()
    assert np.array_equal(np.bincount(s2, minlength=G), np.full(G, E // G))


def test_dispatched_rows_definition():
    idx = np.array([[0, 1], [2, 3], [0, 3]])
    assert P.dispatched_rows(idx, np.array([0, 0, 1, 1])) == 1 + 1 + 2
    assert P.dispatched_rows(idx, np.array([0, 1, 2, 3])) == 6


# ---------------------------------------------------------------- native parity

def _native():
    from routing_dispatch_expert_top_amd import ops
    ops.lib()
    return ops


def _synthetic_stats(wi):
    import oracle
    from routing_dispatch_expert_top_amd import synth
    w = synth.with_shape(synth.workload(wi), T=2048)
    idx, _ = oracle.route(synth.logits(w), w.k, w.n_groups, w.topk_groups)
    coact = oracle.coact(idx, w.E)
    load = np.bincount(idx.ravel(), minlength=w.E)
    return w, idx, coact, load


PARITY = [(1, 1, 8), (2, 1, 8), (2, 4, 8), (2, 8, 0), (3, 1, 2), (3, 8, 8)]


@pytest.mark.parametrize("wi,rpn,passes", PARITY, ids=[f"w{a}_rpn{b}_p{c}" for a, b, c in PARITY])
def test_native_matches_oracle_on_routing_stats(wi, rpn, passes):
    ops = _native()
    w, idx, coact, load = _synthetic_stats(wi)
    G = w.G
    want = P.plan(coact, load, G, rpn, passes)
    got = ops.moe_plan_placement(coact, load, G, rpn, passes)
    assert np.array_equal(got, want)


EDGE = [("G1", 8, 1, 1), ("cap1", 8, 8, 4), ("zeros", 16, 4, 2), ("ties", 16, 4, 4), ("planted", 32, 4, 2)]


@pytest.mark.parametrize("name,E,G,rpn", EDGE, ids=[e[0] for e in EDGE])
def test_native_matches_oracle_edge_cases(name, E, G, rpn):
    ops = _native()
    rng = np.random.default_rng(E * 7 + G)
    if name == "zeros":
        c, load = np.zeros((E, E), np.int64), np.zeros(E, np.int64)
    elif name == "ties":
        c, load = np.full((E, E), 3, np.int64), np.full(E, 5, np.int64)
    elif name == "planted":
        c, load, _ = planted(E, G, 9)
    else:
        c, load = rng.integers(0, 20, (E, E)), rng.integers(0, 20, E)
    assert np.array_equal(ops.moe_plan_placement(c, load, G, rpn, 8), P.plan(c, load, G, rpn, 8))


def test_native_argument_errors():
    ops = _native()
    L = ops.lib()
    c = np.zeros((8, 8), np.int64); ld = np.ones(8, np.int64); pl = np.zeros(8, np.int32)
    args = lambda E, G, rpn, sp: (c.ctypes.data, ld.ctypes.data, E, G, rpn, sp, pl.ctypes.data)
    assert L.moe_plan_placement(*args(8, 3, 1, 1)) == ops.MOE_ERR_ARG      # G does not divide E
    assert L.moe_plan_placement(*args(8, 4, 3, 1)) == ops.MOE_ERR_ARG      # rpn does not divide G
    assert L.moe_plan_placement(*args(8, 4, 1, -1)) == ops.MOE_ERR_ARG
    assert L.moe_plan_placement(None, ld.ctypes.data, 8, 4, 1, 1, pl.ctypes.data) == ops.MOE_ERR_ARG
    ld[3] = -1
    assert L.moe_plan_placement(*args(8, 4, 1, 1)) == ops.MOE_ERR_ARG
