"""Seeded synthetic workloads for the MoE-layer hot path.

This module only draws inputs: router logits, token activations, expert
weights and expert placements. It computes nothing the layer computes (no
routing, no counting, no layout, no FFN), so the fp64 reference and the HIP
library can both be fed from it without sharing any of the layer's arithmetic.

The workload family imitates what the pages report of trained routers:
single tokens tend to select the same expert pairs again and again (Cobalt
page, English abstract), and at top-2 a tiny fraction of the expert pairs
accounts for a large share of the tokens (Zyphra correlated-placement page,
English abstract). Each token draws a latent cluster of experts from a
truncated Zipf law and gets a logit boost on that cluster's members, on top
of N(0,1) noise.

Placements are a partition of E experts over G virtual expert-parallel ranks
(Zyphra page, English abstract: expert parallelism spreads the experts over
GPUs, and correlated placement keeps experts that are often chosen together
on one GPU): ``contiguous`` (expert e on rank e // (E/G)) or ``colocated``
(each latent cluster on one rank).

Activations and weights are drawn in fp32 and rounded to bf16 with
round-to-nearest-even for the bf16 workloads; bf16 arrays are carried as
``uint16`` bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    """Shape and generator recipe of one synthetic MoE-layer workload."""

    name: str
    T: int            # tokens on this GPU
    d: int            # model dim
    E: int            # experts
    k: int            # experts per token
    F: int            # expert FFN hidden dim
    G: int            # virtual expert-parallel ranks
    dtype: str        # activation / weight type: "f32" or "bf16"
    clusters: int     # latent expert clusters (E // clusters experts each)
    zipf: float       # Zipf exponent of the token->cluster law (0 = uniform)
    boost: float      # logit boost on the token's cluster members
    hot_bias: float = 0.0   # extra logit on one expert for every token (load skew)
    n_groups: int = 1       # group-limited routing: contiguous expert groups
    topk_groups: int = 1    # groups kept per token
    note: str = field(default="", compare=False)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def tag(self) -> str:
        s = (f"moe_T{self.T}_d{self.d}_E{self.E}_k{self.k}_F{self.F}_G{self.G}_"
             f"{self.dtype}")
        if self.n_groups > 1:
            s += f"_grp{self.topk_groups}of{self.n_groups}"
        return s


# Hot-expert logit bias for the 8192-token, 128-expert workload. It is the
# largest value on the grid {0, 0.125, ..., 8} for which the busiest expert
# receives at most 8x the mean number of token assignments (the workload asks
# for a per-expert load skewed up to 8x the mean). A CPU test re-derives it
# with the reference router.
HOT_BIAS_T8192 = 1.25

WORKLOADS = [
    Workload("tiny_f32", T=256, d=128, E=8, k=2, F=256, G=4, dtype=F32,
             clusters=4, zipf=0.0, boost=2.0,
             note="4 latent clusters of 2 experts, uniform cluster draw"),
    Workload("top2_E64", T=4096, d=2048, E=64, k=2, F=1408, G=8, dtype=BF16,
             clusters=8, zipf=1.1, boost=2.5),
    Workload("top6_E64", T=4096, d=2048, E=64, k=6, F=1408, G=8, dtype=BF16,
             clusters=8, zipf=1.1, boost=1.5),
    Workload("top8_E128_skew", T=8192, d=4096, E=128, k=8, F=1536, G=16,
             dtype=BF16, clusters=16, zipf=1.2, boost=2.0,
             hot_bias=HOT_BIAS_T8192),
    Workload("top8_E256_grouped", T=16384, d=7168, E=256, k=8, F=2048, G=32,
             dtype=BF16, clusters=32, zipf=1.0, boost=2.0,
             n_groups=8, topk_groups=4),
]

BENCH_WORKLOAD = 3   # the 8192-token, d=4096, 128-expert top-8 layer


def workload(i_or_name) -> Workload:
    if isinstance(i_or_name, int):
        return WORKLOADS[i_or_name]
    for w in WORKLOADS:
        if w.name == i_or_name:
            return w
    raise KeyError(i_or_name)


def custom(**kw) -> Workload:
    """A workload of arbitrary shape built on the tiny recipe's defaults."""
    base = dict(name="custom", T=64, d=64, E=8, k=2, F=64, G=4, dtype=F32,
                clusters=4, zipf=0.0, boost=2.0)
    base.update(kw)
    return Workload(**base)


# --------------------------------------------------------------------------
# bf16 bit helpers (storage conversion of generated inputs)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = u + np.uint32(0x7FFF)
    r += lsb
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return (bf16_bits_to_f32(a) if dtype == BF16 else np.asarray(a, np.float32)).astype(np.float64)


# --------------------------------------------------------------------------
# generator
# --------------------------------------------------------------------------

# Child streams of SeedSequence(seed), by position.
_S_PERM, _S_CLUSTER, _S_NOISE, _S_X, _S_W = range(5)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == BF16 else a32


def cluster_perm(w: Workload, seed: int = 0) -> np.ndarray:
    """Seeded permutation pi of experts; latent cluster c = pi[c*s:(c+1)*s]."""
    ss = np.random.SeedSequence(seed).spawn(5)
    return np.random.Generator(np.random.PCG64(ss[_S_PERM])).permutation(w.E).astype(np.int32)


def placement(w: Workload, kind: str = "contiguous", seed: int = 0) -> np.ndarray:
    """place[E] int32 in [0, G): a partition of the experts over G ranks."""
    E, G = w.E, w.G
    if E % G:
        raise ValueError("placements here need G | E")
    if kind == "contiguous":
        return (np.arange(E, dtype=np.int32) // (E // G)).astype(np.int32)
    if kind == "colocated":
        if w.clusters != G:
            raise ValueError("co-located placement puts one latent cluster per rank")
        pi = cluster_perm(w, seed)
        s = E // w.clusters
        place = np.empty(E, np.int32)
        for c in range(w.clusters):
            place[pi[c * s:(c + 1) * s]] = c
        return place
    raise ValueError(kind)


def replicas(place: np.ndarray, G: int, ranks_per_node: int, copies: int = 2,
             seed: int = 0) -> list:
    """Expert copies for the replica-aware layout: expert e keeps its rank
    place[e] and gets copies - 1 more, each on a different other node (drawn
    with the seed) at the same position inside that node. Cobalt page,
    English abstract: expert replicas are spread over GPUs of several nodes;
    how many and where is not stated, so this is a synthetic choice."""
    nodes = G // ranks_per_node
    rng = np.random.default_rng(seed)
    out = []
    for p in np.asarray(place).astype(np.int64):
        home_node, pos = divmod(int(p), ranks_per_node)
        others = [n for n in range(nodes) if n != home_node]
        extra = rng.permutation(others)[:max(0, min(copies, nodes) - 1)] if others else []
        out.append(sorted([int(p)] + [int(n) * ranks_per_node + pos for n in extra]))
    return out


def replica_masks(reps) -> np.ndarray:
    """Per-expert rank lists -> [E] uint32 bit masks (bit g: rank g)."""
    m = np.zeros(len(reps), np.uint32)
    for e, rs in enumerate(reps):
        for g in rs:
            m[e] |= np.uint32(1) << np.uint32(g)
    return m


def _batch_streams(seed: int, batch: int):
    """Seed streams of the per-token draws. The model structure (expert
    clusters, cross-layer maps) depends on ``seed`` only; ``batch`` > 0 draws
    another batch of tokens from the same model (batch 0 is the default one)."""
    if batch == 0:
        return np.random.SeedSequence(seed).spawn(5)
    return np.random.SeedSequence([seed, 1000 + batch]).spawn(5)


def token_clusters(w: Workload, seed: int = 0, batch: int = 0) -> np.ndarray:
    ss = _batch_streams(seed, batch)
    rng = np.random.Generator(np.random.PCG64(ss[_S_CLUSTER]))
    C = w.clusters
    if w.zipf > 0:
        p = (np.arange(1, C + 1, dtype=np.float64)) ** (-w.zipf)
        p /= p.sum()
    else:
        p = np.full(C, 1.0 / C)
    return rng.choice(C, size=w.T, p=p).astype(np.int32)


def logits(w: Workload, seed: int = 0, hot_bias: float | None = None,
           batch: int = 0) -> np.ndarray:
    """Router logits [T, E] fp32: N(0,1) + boost on the token's cluster."""
    ss = _batch_streams(seed, batch)
    rng = np.random.Generator(np.random.PCG64(ss[_S_NOISE]))
    L = rng.standard_normal((w.T, w.E), dtype=np.float32)
    pi = cluster_perm(w, seed)
    s = w.E // w.clusters
    members = pi.reshape(w.clusters, s)                 # [C, s]
    tc = token_clusters(w, seed, batch)
    rows = np.repeat(np.arange(w.T), s)
    cols = members[tc].reshape(-1)
    L[rows, cols] += np.float32(w.boost)
    hb = w.hot_bias if hot_bias is None else hot_bias
    if hb:
        L[:, pi[0]] += np.float32(hb)
    return L


def next_layer_logits(w: Workload, seed: int = 0, follow: float = 0.8,
                      batch: int = 0) -> np.ndarray:
    """Router logits [T, E] of the following MoE layer, correlated with this
    layer's (Zyphra page, English abstract: the experts a token selects at one
    layer predict those it selects at the next). The next layer has its own
    latent clusters (a fresh expert permutation); token t's next-layer
    cluster is sigma(c_t), sigma a seeded permutation of the clusters and c_t
    its cluster here, with probability ``follow``, else a fresh draw from the
    same Zipf law. Noise, boost and hot bias as in :func:`logits`; ``batch``
    as there (same model, other tokens)."""
    ss = np.random.SeedSequence([seed, 1]).spawn(4)
    if batch:
        ss = ss[:1] + np.random.SeedSequence([seed, 1, 1000 + batch]).spawn(3)
    g = [np.random.Generator(np.random.PCG64(x)) for x in ss]
    C, s = w.clusters, w.E // w.clusters
    pi2 = g[0].permutation(w.E).astype(np.int32)
    sigma = g[0].permutation(C)
    if w.zipf > 0:
        p = (np.arange(1, C + 1, dtype=np.float64)) ** (-w.zipf)
        p /= p.sum()
    else:
        p = np.full(C, 1.0 / C)
    tc = token_clusters(w, seed, batch)
    fresh = g[1].choice(C, size=w.T, p=p)
    keep = g[1].random(w.T) < follow
    tc2 = np.where(keep, sigma[tc], fresh)
    L = g[2].standard_normal((w.T, w.E), dtype=np.float32)
    members = pi2.reshape(C, s)
    rows = np.repeat(np.arange(w.T), s)
    L[rows, members[tc2].reshape(-1)] += np.float32(w.boost)
    if w.hot_bias:
        L[:, pi2[0]] += np.float32(w.hot_bias)
    return L


def activations(w: Workload, seed: int = 0) -> np.ndarray:
    """Token activations x [T, d]: N(0,1), stored in the workload dtype."""
    ss = np.random.SeedSequence(seed).spawn(5)
    rng = np.random.Generator(np.random.PCG64(ss[_S_X]))
    return _store(rng.standard_normal((w.T, w.d), dtype=np.float32), w.dtype)


def _expert_seeds(w: Workload, seed: int):
    ss = np.random.SeedSequence(seed).spawn(5)
    return ss[_S_W].spawn(3 * w.E)   # [gate e, up e, down e] interleaved


def weights(w: Workload, seed: int = 0, experts=None):
    """Expert weights W_gate, W_up [E, F, d] and W_down [E, d, F] (out x in).

    Entries are N(0, 1/fan_in) (fan_in = d for gate/up, F for down), stored
    in the workload dtype. ``experts`` restricts generation to a subset (the
    other rows are left zero); each expert has its own seed stream, so a
    subset draws exactly the values of the full set.
    """
    E, F, d = w.E, w.F, w.d
    st = np.uint16 if w.dtype == BF16 else np.float32
    wg = np.zeros((E, F, d), st)
    wu = np.zeros((E, F, d), st)
    wd = np.zeros((E, d, F), st)
    seeds = _expert_seeds(w, seed)
    todo = range(E) if experts is None else sorted(set(int(e) for e in experts))
    sg, sd = np.float32(1.0 / np.sqrt(d)), np.float32(1.0 / np.sqrt(F))

    def one(job):
        e, which = job
        rng = np.random.Generator(np.random.PCG64(seeds[3 * e + which]))
        if which < 2:
            a = rng.standard_normal((F, d), dtype=np.float32)
            a *= sg
            (wg if which == 0 else wu)[e] = _store(a, w.dtype)
        else:
            a = rng.standard_normal((d, F), dtype=np.float32)
            a *= sd
            wd[e] = _store(a, w.dtype)

    jobs = [(e, j) for e in todo for j in range(3)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, jobs))
    return wg, wu, wd


def make(w: Workload, seed: int = 0, place: str = "contiguous", with_weights: bool = True):
    """All inputs of one layer call as host numpy arrays."""
    out = dict(logits=logits(w, seed), x=activations(w, seed),
               place=placement(w, place, seed))
    if with_weights:
        out["w_gate"], out["w_up"], out["w_down"] = weights(w, seed)
    return out


def with_shape(w: Workload, **kw) -> Workload:
    return replace(w, **kw)
