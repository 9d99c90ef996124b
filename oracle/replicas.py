"""TEST INFRASTRUCTURE: plain reference of replica-aware dispatch assignment.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use
this. It shares no code with the library's kernels.

Cobalt page, English abstract: expert replicas sit on GPUs of several nodes,
and a communication-aware task assignment routes each token to fewer remote
nodes given the current expert layout; cross-node token traffic falls. The
pages give no algorithm; the reading implemented (and followed by the
library) is a greedy cover per token:

  ranks are grouped into nodes of `rpn` consecutive ranks; token t's home
  rank is t * G // T (tokens sharded contiguously over the ranks) and its
  home node that rank's node. Among the token's valid choices j (expert in
  [0, E) with at least one replica):
  nodes  : while choices remain, take the node holding a replica of the most
           remaining choices (ties: the home node, then the lowest node) and
           give it every remaining choice it can serve;
  ranks  : inside each node so chosen (in the order chosen), while its
           choices remain, take the rank of that node holding the most of
           them (ties: the home rank, then the lowest rank) and give it every
           remaining choice it can serve.

The layout built from the per-choice ranks follows the once-per-rank
dispatcher of the Zyphra page (English abstract) exactly as the placement
layout does: rows rank by rank, tokens ascending within a rank; slots expert
by expert, tokens ascending within an expert.
"""
from __future__ import annotations

import numpy as np


def reps_from_mask(rep_mask, G: int) -> list:
    """rep_mask[e] bit g set iff rank g < G holds a copy of expert e ->
    per-expert sorted rank lists."""
    return [[g for g in range(G) if (int(m) >> g) & 1] for m in np.asarray(rep_mask).astype(np.int64)]


def assign(topk_idx, reps, G: int, rpn: int) -> np.ndarray:
    """reps[e] = ranks holding a copy of expert e.
    -> rank_of [T, k] int32 (-1 where the choice is invalid)."""
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    E = len(reps)
    reps = [sorted(set(int(r) for r in rs if 0 <= int(r) < G)) for rs in reps]
    rank_of = np.full((T, k), -1, dtype=np.int32)
    nodes = G // rpn
    for t in range(T):
        home = t * G // T
        hnode = home // rpn
        left = [j for j in range(k) if 0 <= idx[t, j] < E and reps[idx[t, j]]]
        order = []
        node_of = {}
        while left:
            def served(n):
                return [j for j in left if any(r // rpn == n for r in reps[idx[t, j]])]
            best = max(range(nodes), key=lambda n: (len(served(n)), n == hnode, -n))
            for j in served(best):
                node_of[j] = best
            left = [j for j in left if j not in node_of]
            order.append(best)
        for n in order:
            mine = [j for j in range(k) if node_of.get(j) == n]
            while mine:
                def held(r):
                    return [j for j in mine if r in reps[idx[t, j]]]
                best = max(range(n * rpn, (n + 1) * rpn), key=lambda r: (len(held(r)), r == home, -r))
                for j in held(best):
                    rank_of[t, j] = best
                mine = [j for j in mine if rank_of[t, j] < 0]
    return rank_of


def layout(topk_idx, rank_of, E: int, G: int) -> dict:
    """Once-per-rank layout from per-choice ranks (same outputs and orders as
    the placement layout; invalid choices, rank -1, get no slot)."""
    idx = np.asarray(topk_idx).astype(np.int64)
    ro = np.asarray(rank_of).astype(np.int64)
    T, k = idx.shape
    valid = ro >= 0
    rank_mask = np.zeros(T, np.uint64)
    for j in range(k):
        rank_mask |= np.where(valid[:, j], np.uint64(1) << np.maximum(ro[:, j], 0).astype(np.uint64),
                              np.uint64(0))
    rank_mask = rank_mask.astype(np.uint32)
    # rows: rank by rank, tokens ascending within a rank
    row_of = np.full((T, G), -1, np.int64)
    disp_token, rank_off, r = [], [0], 0
    for g in range(G):
        toks = np.flatnonzero((rank_mask >> np.uint32(g)) & np.uint32(1))
        row_of[toks, g] = r + np.arange(len(toks))
        disp_token.extend(toks.tolist())
        r += len(toks)
        rank_off.append(r)
    # slots: expert by expert, tokens ascending within an expert (then choice)
    t_of, j_of = np.nonzero(valid)
    e_of = idx[t_of, j_of]
    order = np.lexsort((j_of, t_of, e_of))
    t_s, j_s, e_s = t_of[order], j_of[order], e_of[order]
    expert_off = np.concatenate([[0], np.cumsum(np.bincount(e_s, minlength=E))]).astype(np.int32)
    perm_row = row_of[t_s, ro[t_s, j_s]].astype(np.int32)
    slot_of = np.full(T * k, -1, np.int32)
    slot_of[t_s * k + j_s] = np.arange(len(order), dtype=np.int32)
    return dict(rank_mask=rank_mask, rank_off=np.array(rank_off, np.int32),
                disp_token=np.array(disp_token, np.int32), expert_off=expert_off,
                perm_row=perm_row, slot_of=slot_of, R=r)


def node_stats(rank_mask, G: int, rpn: int) -> dict:
    """Per token: node_mask (bit n if a row goes to a rank of node n). Totals:
    rows to ranks outside the token's home node, and remote nodes reached
    (the transfers a node-level dedup would make)."""
    T = len(rank_mask)
    node_mask = np.zeros(T, np.uint32)
    cross_rows = cross_nodes = 0
    for t in range(T):
        hnode = (t * G // T) // rpn
        for g in range(G):
            if (int(rank_mask[t]) >> g) & 1:
                node_mask[t] |= np.uint32(1) << np.uint32(g // rpn)
                cross_rows += (g // rpn) != hnode
        for n in range(G // rpn):
            cross_nodes += ((int(node_mask[t]) >> n) & 1) and n != hnode
    return dict(node_mask=node_mask, cross_node_rows=int(cross_rows),
                cross_node_transfers=int(cross_nodes))
