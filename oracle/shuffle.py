"""TEST INFRASTRUCTURE: plain reference of token shuffling and the
token-locality statistic.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use
this. It shares no code with the library's kernels.

Source: Zyphra correlated expert placement page, English abstract (token
shuffling under sequence parallelism; the page reports the on-GPU share of
assignments going from 12.5% to 59% on one node). Reading: a token should sit
on the GPU that will serve most of its next-layer experts, and 12.5% is 1/8,
the share uniform routing gives on 8 GPUs. The pages give no rule for the
prediction or the choice of GPU; the reading implemented (and followed by
the library) is:

  home rank of token t: t * G // T (tokens sharded in order);
  prediction model: an affinity table aff [E, G] >= 0, aff[e][g] = how
    strongly a token using expert e now is expected to need rank g next
    (e.g. cross-layer co-activation counts summed over the next layer's
    experts on g; a one-hot table of a placement gives "the rank holding the
    most of these experts");
  destination: the rank g maximising sum_j aff[want[t, j]][g] over the
    token's valid experts (0 <= want < E; ties: the home rank, then the
    lowest rank);
  shuffled order: tokens grouped by destination rank, ascending within a
    rank (a stable sort), with per-rank offsets and the inverse permutation.

The locality statistic is the share of (token, choice) pairs whose expert
sits on the rank that holds the token.
"""
from __future__ import annotations

import numpy as np


def home_ranks(T: int, G: int) -> np.ndarray:
    return (np.arange(T, dtype=np.int64) * G // T).astype(np.int32) if T else np.zeros(0, np.int32)


def onehot(place, G: int) -> np.ndarray:
    """aff[e][g] = 1 if expert e sits on rank g."""
    place = np.asarray(place)
    aff = np.zeros((len(place), G), np.int64)
    aff[np.arange(len(place)), place] = 1
    return aff


def destinations(want_idx, aff, G: int) -> np.ndarray:
    want = np.asarray(want_idx)
    T, k = want.shape
    aff = np.asarray(aff, np.int64)
    E = aff.shape[0]
    dest = np.empty(T, np.int32)
    for t in range(T):
        home = t * G // T
        score = [0] * G
        for j in range(k):
            e = int(want[t, j])
            if 0 <= e < E:
                for g in range(G):
                    score[g] += int(aff[e, g])
        dest[t] = max(range(G), key=lambda r: (score[r], r == home, -r))
    return dest


def shuffle(dest, G: int) -> dict:
    """-> perm (tokens in shuffled order), rank_off [G+1], pos (inverse)."""
    dest = np.asarray(dest, np.int64)
    perm = np.argsort(dest, kind="stable").astype(np.int32)
    rank_off = np.concatenate([[0], np.cumsum(np.bincount(dest, minlength=G))]).astype(np.int32)
    pos = np.empty(len(dest), np.int32)
    pos[perm] = np.arange(len(dest), dtype=np.int32)
    return dict(perm=perm, rank_off=rank_off, pos=pos)


def local_share(topk_idx, place, token_rank) -> float:
    """Share of (t, j) with place[topk_idx[t, j]] == token_rank[t]."""
    idx = np.asarray(topk_idx)
    if idx.size == 0:
        return 0.0
    ranks = np.asarray(place)[idx]
    return float((ranks == np.asarray(token_rank)[:, None]).mean())
