"""TEST INFRASTRUCTURE: plain reference of the expert placement planner.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use
this. It shares no code with the library's planner.

Cobalt page, English abstract: a two-stage layout planner periodically
co-locates frequently co-activated experts and adjusts the layout inside each
node every step to rebalance the workload. Zyphra correlated expert placement
page, English abstract: experts often selected together are put on the same
GPU, so the once-per-GPU dispatcher sends fewer rows.

The pages give no algorithm; the reading implemented (and the one the
library follows) is:

stage 1 (co-location, E/G experts per rank)
  for g = 0..G-1: seed = heaviest unassigned expert (load; ties: lowest
  index); then, until the group holds E/G experts, add the unassigned expert
  with the largest summed weight to the group's members (ties: larger load,
  then lowest index). Then up to `swap_passes` passes: for a = 0..E-1, for
  b = a+1..E-1, if a and b sit in different groups and swapping them raises
  the total within-group weight W, swap (at once; later pairs see the new
  groups). A pass without a swap ends stage 1.

stage 2 (per-node rebalance, only if ranks_per_node > 1)
  node n = ranks [n*rpn, (n+1)*rpn). Repeat per node: h = most loaded rank,
  l = least loaded (ties: lowest rank); stop if equal. Among expert pairs
  (a on h, b on l, load[a] > load[b]) whose swap makes
  max(L[h] - d, L[l] + d) < L[h] (d = load[a] - load[b]), take the one with
  the smallest such maximum, then the largest change of W, then lowest a,
  then lowest b; stop if there is none.

Weights: w(a, b) = coact[a][b] + coact[b][a] for a != b, w(a, a) = 0.
"""
from __future__ import annotations

import numpy as np


def weights(coact: np.ndarray) -> np.ndarray:
    c = np.asarray(coact, dtype=np.int64)
    w = c + c.T
    np.fill_diagonal(w, 0)
    return w


def within_weight(w: np.ndarray, place: np.ndarray) -> int:
    """W = sum over unordered pairs (a, b) on the same rank of w(a, b)."""
    same = place[:, None] == place[None, :]
    return int(np.triu(w * same, 1).sum())


def swap_delta(w: np.ndarray, place: np.ndarray, a: int, b: int) -> int:
    """W after swapping the ranks of a and b, minus W before (full recount)."""
    p = place.copy()
    p[a], p[b] = p[b], p[a]
    return within_weight(w, p) - within_weight(w, place)


def stage1(w: np.ndarray, load: np.ndarray, G: int, swap_passes: int) -> np.ndarray:
    E = len(load)
    cap = E // G
    place = np.full(E, -1, dtype=np.int64)
    for g in range(G):
        free = [e for e in range(E) if place[e] < 0]
        seed = max(free, key=lambda e: (load[e], -e))
        members = [seed]
        place[seed] = g
        while len(members) < cap:
            free = [e for e in range(E) if place[e] < 0]
            u = max(free, key=lambda e: (int(w[e, members].sum()), load[e], -e))
            members.append(u)
            place[u] = g
    for _ in range(swap_passes):
        swapped = False
        for a in range(E):
            for b in range(a + 1, E):
                if place[a] != place[b] and swap_delta(w, place, a, b) > 0:
                    place[a], place[b] = place[b], place[a]
                    swapped = True
        if not swapped:
            break
    return place


def stage2(w: np.ndarray, load: np.ndarray, place: np.ndarray, G: int, rpn: int) -> np.ndarray:
    place = place.copy()
    E = len(load)
    for n0 in range(0, G, rpn):
        ranks = list(range(n0, n0 + rpn))
        while True:
            L = {r: int(load[place == r].sum()) for r in ranks}
            h = max(ranks, key=lambda r: (L[r], -r))
            l = min(ranks, key=lambda r: (L[r], r))
            if L[h] == L[l]:
                break
            best = None
            for a in range(E):
                if place[a] != h:
                    continue
                for b in range(E):
                    if place[b] != l:
                        continue
                    d = int(load[a] - load[b])
                    if d <= 0:
                        continue
                    nm = max(L[h] - d, L[l] + d)
                    if nm >= L[h]:
                        continue
                    key = (nm, -swap_delta(w, place, a, b), a, b)
                    if best is None or key < best:
                        best = key
            if best is None:
                break
            a, b = best[2], best[3]
            place[a], place[b] = place[b], place[a]
    return place


def plan(coact, load, G: int, ranks_per_node: int = 1, swap_passes: int = 8) -> np.ndarray:
    """-> place [E] int32 (rank of each expert)."""
    load = np.asarray(load, dtype=np.int64)
    E = len(load)
    if E % G or G % ranks_per_node:
        raise ValueError("need G | E and ranks_per_node | G")
    w = weights(coact)
    place = stage1(w, load, G, swap_passes)
    if ranks_per_node > 1:
        place = stage2(w, load, place, G, ranks_per_node)
    return place.astype(np.int32)


def dispatched_rows(topk_idx: np.ndarray, place: np.ndarray) -> int:
    """R = number of distinct (token, rank) pairs: the rows a once-per-rank
    dispatcher sends (Zyphra page, English abstract)."""
    ranks = np.asarray(place)[np.asarray(topk_idx)]
    ranks = np.sort(ranks, axis=1)
    return int(ranks.shape[0] + (np.diff(ranks, axis=1) != 0).sum())


def rank_loads(load, place, G: int) -> np.ndarray:
    return np.bincount(np.asarray(place), weights=np.asarray(load, dtype=np.float64),
                       minlength=G).astype(np.int64)
