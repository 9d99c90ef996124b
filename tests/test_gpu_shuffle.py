"""GPU parity of token shuffling (moe_token_shuffle) against the reference:
bit-exact destinations, per-rank offsets, the shuffled order, its inverse
and the shuffled rows."""
import numpy as np
import pytest
import torch

import oracle
from oracle import shuffle as sh
from routing_dispatch_expert_top_amd import ops, synth
from tests.gpu_helpers import dev, host
from tests.test_shuffle import load_golden

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()


def run_shuffle(want, aff, x=None):
    out = ops.moe_token_shuffle(dev(np.ascontiguousarray(want, np.int32)),
                                dev(np.ascontiguousarray(aff, np.int32)),
                                dev(x) if x is not None else None)
    torch.cuda.synchronize()
    g = {key: host(out[key]) for key in ("dest", "rank_off", "perm", "pos")}
    if x is not None:
        g["x_shuf"] = host(out["x_shuf"])
    return g


def check(g, want, aff, G, x=None):
    dest = sh.destinations(want, aff, G)
    r = sh.shuffle(dest, G)
    assert np.array_equal(g["dest"], dest)
    for key in ("rank_off", "perm", "pos"):
        assert np.array_equal(g[key], r[key]), key
    if x is not None:
        assert np.array_equal(g["x_shuf"], oracle.dispatch_rows(x, r["perm"]))


CASES = [  # T, E, k, G, table, dtype, d, seed
    (777, 16, 4, 8, "onehot", "bf16", 256, 0),
    (1, 8, 2, 4, "counts", "bf16", 64, 1),
    (2049, 64, 6, 3, "counts", "f32", 128, 2),
    (500, 32, 8, 32, "counts", None, 0, 3),
    (300, 128, 16, 16, "signed", "bf16", 64, 4),
    (64, 4, 1, 1, "counts", "f32", 64, 5),
    (1000, 24, 5, 12, "onehot", None, 0, 6),
]


@pytest.mark.parametrize("T,E,k,G,table,dtype,d,seed", CASES)
def test_shuffle_parity(T, E, k, G, table, dtype, d, seed):
    print(f"case shuffle T={T} E={E} k={k} G={G} {table}", flush=True)
    rng = np.random.default_rng(seed)
    want = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    want[rng.random((T, k)) < 0.05] = -1                     # not an expert
    want[rng.random((T, k)) < 0.02] = E + 3
    if table == "onehot":
        aff = sh.onehot(rng.integers(0, G, size=E), G)
    elif table == "counts":
        aff = rng.integers(0, 5, size=(E, G))
    else:
        aff = rng.integers(-(1 << 30), 1 << 30, size=(E, G))   # large, both signs: int64 sums
    x = None
    if dtype is not None:
        x32 = rng.standard_normal((T, d)).astype(np.float32)
        x = synth.f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    g = run_shuffle(want, aff, x)
    check(g, want, aff, G, x)


@pytest.mark.parametrize("name", ["A", "B"])
def test_shuffle_golden(name):
    c = load_golden()[name]
    aff = (np.array(c["aff"]).reshape(c["E"], c["G"]) if "aff" in c
           else sh.onehot(c["place"], c["G"]))
    g = run_shuffle(c["want"], aff)
    for key in ("dest", "perm", "rank_off", "pos"):
        assert g[key].tolist() == c[key], key


def test_empty_batch():
    g = run_shuffle(np.zeros((0, 2), np.int32), np.ones((4, 3), np.int32))
    assert g["rank_off"].tolist() == [0, 0, 0, 0]


def test_argument_errors():
    want = dev(np.zeros((8, 2), np.int32))
    with pytest.raises(ops.MoeError):
        ops.moe_token_shuffle(want, dev(np.ones((4, 33), np.int32)))   # G > 32
    x = torch.zeros((8, 3), dtype=torch.float32, device="cuda")      # rows not 16-byte multiples
    with pytest.raises(ops.MoeError):
        ops.moe_token_shuffle(want, dev(np.ones((4, 2), np.int32)), x)


@pytest.mark.timeout(300)
def test_full_size_shuffle():
    """T=8192, E=128, k=8, G=16: this layer's routing of the clustered
    logits, a cross-layer affinity table from another batch of the same
    model, and the bf16 rows."""
    w = synth.workload(3)
    print(f"case shuffle full {w.tag()}", flush=True)
    idx, _ = oracle.route(synth.logits(w), w.k)
    c1, _ = oracle.route(synth.logits(w, batch=1), w.k)
    c2, _ = oracle.route(synth.next_layer_logits(w, batch=1), w.k)
    X = np.zeros((w.E, w.E), np.int64)
    for j in range(w.k):
        for j2 in range(w.k):
            np.add.at(X, (c1[:, j], c2[:, j2]), 1)
    aff = X @ sh.onehot(synth.placement(w, "contiguous"), w.G)
    x = synth.activations(w)
    g = run_shuffle(idx, aff, x)
    check(g, idx, aff, w.G, x)
