"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Bit-exact: top-k indices, co-activation counts, rank masks, row and slot
offsets, the row and slot permutations, R and the dispatched rows.
Tolerance (max|gpu-ref| <= tau * max|ref| per tensor): gates 1e-4; h, y and
out 1e-4 in fp32 and 2e-2 in bf16.

Small shapes are checked element by element on every output; they span
several tiles with ragged tails, empty experts, k = 1, k = E, the largest
E / k / G, an odd E, -inf logits and an empty batch. The five workload shapes
are run at full size in the same launch configuration as the benchmark; there
the integer outputs and the dispatched rows are compared in full, h, y and
out in full for the first four, and for the largest (T=16384, d=7168, E=256)
h and y on one slot of every 32-row band of every expert plus out on a token
sample, each evaluated by the oracle on its own.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_dispatch_expert_top_amd import ops, synth
from tests.gpu_helpers import (TAU, TAU_GATES, DevInputs, assert_close, compare_exact, dev, host,
                               run_layer, widen)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()


def C(name, **kw):
    return synth.custom(name=name, **kw)


SMALL = [
    (synth.workload(0), "contiguous"),
    (C("bf16_ragged", T=777, d=256, E=16, k=4, F=192, G=4, dtype="bf16", clusters=4, zipf=1.1,
       boost=2.0), "colocated"),
    (C("f32_ragged", T=500, d=192, E=12, k=3, F=320, G=3, dtype="f32", clusters=3), "contiguous"),
    (C("bf16_grouped", T=300, d=128, E=32, k=4, F=128, G=8, dtype="bf16", clusters=8,
       n_groups=4, topk_groups=2), "colocated"),
    (C("bf16_k_eq_E", T=200, d=128, E=8, k=8, F=128, G=2, dtype="bf16", clusters=2), "contiguous"),
    (C("bf16_k1", T=333, d=128, E=8, k=1, F=64, G=4, dtype="bf16"), "contiguous"),
    (C("bf16_T1", T=1, d=64, E=4, k=2, F=64, G=2, dtype="bf16", clusters=2), "contiguous"),
    (C("bf16_sparse_experts", T=20, d=128, E=64, k=2, F=128, G=8, dtype="bf16", clusters=8),
     "colocated"),
    (C("bf16_max_E_k_G", T=150, d=64, E=256, k=16, F=64, G=32, dtype="bf16", clusters=32),
     "colocated"),
    (C("bf16_odd_E", T=97, d=64, E=5, k=3, F=64, G=1, dtype="bf16", clusters=1), "contiguous"),
    (C("bf16_hot_rows", T=2000, d=128, E=8, k=2, F=128, G=4, dtype="bf16", clusters=4,
       hot_bias=6.0), "colocated"),
]


@pytest.mark.parametrize("w,kind", SMALL, ids=[f"{w.name}-{k}" for w, k in SMALL])
def test_layer_parity_small(w, kind):
    print(f"case {w.name} {w.tag()} {kind}", flush=True)
    inp = synth.make(w, place=kind)
    ref = oracle.layer(inp["logits"], inp["x"], inp["place"], w.G, w.k, inp["w_gate"],
                       inp["w_up"], inp["w_down"], w.n_groups, w.topk_groups, want_h=True)
    g = run_layer(w, DevInputs(w, inp))
    assert g["R"] == ref["R"] and g["S"] == w.T * w.k
    compare_exact(g, ref)
    assert np.array_equal(g["x_disp"], ref["x_disp"])
    assert_close("gates", g["gates"], ref["gates"], TAU_GATES)
    np.testing.assert_allclose(widen(g["gates"]).sum(1), 1.0, atol=1e-6)
    tau = TAU[w.dtype]
    assert_close("h", g["h"], ref["h"], tau)
    assert_close("y", g["y"], ref["y"], tau)
    assert_close("out", g["out"], ref["out"], tau)


def test_layer_parity_neg_inf_logits():
    """-inf router logits act as masks (each token keeps at least k finite
    logits): the masked experts are never chosen and the whole layer still
    matches the oracle."""
    w = C("bf16_neg_inf", T=700, d=128, E=16, k=4, F=128, G=4, dtype="bf16", clusters=4)
    inp = synth.make(w, place="colocated")
    rng = np.random.default_rng(17)
    mask = rng.random((w.T, w.E)) < 0.4
    mask[np.arange(w.T)[:, None], np.argsort(rng.random((w.T, w.E)), 1)[:, :w.k]] = False
    mask[5] = True
    mask[5, :w.k] = False                      # exactly k finite logits
    logits = inp["logits"].copy()
    logits[mask] = -np.inf
    inp = dict(inp, logits=logits)
    ref = oracle.layer(logits, inp["x"], inp["place"], w.G, w.k, inp["w_gate"], inp["w_up"],
                       inp["w_down"], want_h=True)
    g = run_layer(w, DevInputs(w, inp))
    assert not mask[np.arange(w.T)[:, None], g["topk_idx"]].any()
    compare_exact(g, ref)
    assert np.array_equal(g["x_disp"], ref["x_disp"])
    assert_close("gates", g["gates"], ref["gates"], TAU_GATES)
    for key in ("h", "y", "out"):
        assert_close(key, g[key], ref[key], TAU["bf16"])


def test_empty_batch():
    w = C("empty", T=0, d=64, E=8, k=2, F=64, G=4, dtype="bf16")
    lay = ops.Layer(0, 64, 8, 2, 64, 4, torch.bfloat16, "cuda")
    logits = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    place = dev(synth.placement(w))
    wg = torch.zeros((8, 64, 64), dtype=torch.bfloat16, device="cuda")
    lay.lay["rank_off"].fill_(-7)
    lay.lay["expert_off"].fill_(-7)
    lay.forward(logits, x, place, wg, wg, wg)
    torch.cuda.synchronize()
    assert not host(lay.lay["rank_off"]).any() and not host(lay.lay["expert_off"]).any()
    assert not host(lay.coact).any()


def test_coact_accumulates_and_repeats_bit_exactly():
    """Ten passes of the layer on the same inputs: the histogram holds ten
    times the counts and every other output is bit-identical each time (the
    race check: no result may depend on the order of atomics or of waves)."""
    w = synth.with_shape(synth.workload(2), T=1024)
    inp = synth.make(w, place="colocated")
    d_in = DevInputs(w, inp)
    dt = torch.bfloat16
    lay = ops.Layer(w.T, w.d, w.E, w.k, w.F, w.G, dt, "cuda")
    outs = []
    for _ in range(10):
        lay.forward(d_in.logits, d_in.x, d_in.place, d_in.w_gate, d_in.w_up, d_in.w_down)
        torch.cuda.synchronize()
        outs.append({k: host(v).copy() for k, v in
                     dict(out=lay.out, y=lay.y, h=lay.h, perm=lay.lay["perm_row"],
                          slot=lay.lay["slot_of"], tok=lay.lay["disp_token"]).items()})
    ref_c = oracle.coact(oracle.route(inp["logits"], w.k)[0], w.E)
    assert np.array_equal(host(lay.coact).astype(np.int64), 10 * ref_c)
    for o in outs[1:]:
        for key in o:
            assert np.array_equal(o[key], outs[0][key]), key


# (T, E, k, offset): the first eight stay under the row-owner kernel's E*T*k
# bound of 2^26 (one with the routing result 4 bytes off 16-byte alignment,
# which takes its scalar-load variant; E = 4 and E = 2, whose workgroups see
# thousands of hits each, more than their LDS hit queue holds), the last two
# exceed it and take the LDS-triangle kernel; skewed draws make some cells
# hot.
COACT_SHAPES = [(3000, 64, 6, 0), (8192, 128, 8, 0), (2501, 48, 5, 1), (1 << 21, 4, 2, 0),
                (1 << 22, 2, 2, 0), (50000, 64, 6, 0), (20000, 256, 8, 0), (9000, 256, 16, 0),
                (40000, 256, 8, 0), (80000, 128, 8, 0)]


@pytest.mark.parametrize("T,E,k,off", COACT_SHAPES,
                         ids=[f"T{t}_E{e}_k{k}_off{o}" for t, e, k, o in COACT_SHAPES])
def test_coact_both_kernels(T, E, k, off):
    print(f"case coact T={T} E={E} k={k} offset={off}", flush=True)
    rng = np.random.default_rng(T * 1000 + E + k)
    score = rng.random((T, E)) + np.linspace(0.0, 0.6, E)[None, :]
    idx = np.argsort(-score, axis=1)[:, :k].astype(np.int32)
    ref = oracle.coact(idx, E)
    seed = rng.integers(0, 5, size=(E, E)).astype(np.int32)
    seed = seed + seed.T
    buf = torch.empty(T * k + off, dtype=torch.int32, device="cuda")
    buf[off:] = dev(idx.reshape(-1))
    got = ops.moe_coact_hist(buf[off:].view(T, k), E, coact=dev(seed))
    torch.cuda.synchronize()
    assert np.array_equal(host(got).astype(np.int64) - seed, ref)


# (E, n_groups, topk_groups, k): groups of 4 to 128 experts (1 to 32 lanes of
# 4 logits each, where a group's maximum is a reduction over its own lanes),
# groups of 6 and 12 experts (a lane's logits in two groups; 3 lanes per
# group), and 2 to 64 lanes per token.
ROUTE_GROUPS = [(16, 4, 2, 3), (32, 4, 2, 4), (64, 8, 3, 6), (128, 4, 2, 8), (256, 8, 4, 8),
                (256, 4, 1, 8), (256, 2, 1, 16), (36, 6, 3, 5), (48, 4, 3, 7), (8, 2, 1, 2)]


@pytest.mark.parametrize("E,ng,tg,k", ROUTE_GROUPS,
                         ids=[f"E{e}_g{g}_top{t}_k{k}" for e, g, t, k in ROUTE_GROUPS])
def test_route_group_limited(E, ng, tg, k):
    """Group-limited top-k, bit-exact indices: a third of the rows on a coarse
    grid (tied logits and tied group maxima), some signed zeros, a ragged T."""
    print(f"case route E={E} groups={ng} top_groups={tg} k={k}", flush=True)
    rng = np.random.default_rng(E * 100 + ng * 10 + tg)
    T = 3001
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[::3] = np.round(logits[::3] * 2.0) / 2.0
    logits[1::7, 0] = -0.0
    # -inf masks: in rows 2, 7, 12, ... one expert per group, so every group
    # keeps a finite maximum and the chosen groups hold at least k finite
    # logits (tg * (E/ng - 1) >= k for every case listed)
    gs = E // ng
    assert tg * (gs - 1) >= k
    rows = np.arange(2, T, 5)
    cols = (np.arange(ng)[None, :] * gs + (rows[:, None] % gs))
    logits[rows[:, None], cols] = -np.inf
    idx_ref, g_ref = oracle.route(logits, k, ng, tg)
    assert np.isfinite(g_ref).all()
    idx, gates = ops.moe_route(dev(logits), k, ng, tg)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), idx_ref)
    assert_close("gates", host(gates), g_ref, TAU_GATES)


def test_combine_identity_experts_returns_input():
    """With y = the token's own row (identity experts), out = x up to rounding."""
    w = synth.with_shape(synth.workload(2), T=1500)
    inp = synth.make(w, place="colocated", with_weights=False)
    idx, gates = oracle.route(inp["logits"], w.k)
    lay = oracle.layout(idx, w.E, inp["place"], w.G)
    y = inp["x"][lay["disp_token"][lay["perm_row"]]]          # bf16 bits, slot order
    g32 = gates.astype(np.float32)
    out = ops.moe_combine(dev(y), dev(lay["slot_of"]), dev(g32), w.T, w.k)
    torch.cuda.synchronize()
    x = widen(inp["x"])
    ref = oracle.combine(widen(y), lay["slot_of"], g32.astype(np.float64), w.T, w.k)
    assert_close("out", host(out), ref, 2.0 ** -8)
    assert_close("out_vs_x", host(out), x, 2.0 ** -8)


def test_ffn_alone_on_oracle_layout():
    w = C("ffn_only", T=640, d=192, E=6, k=2, F=256, G=3, dtype="bf16", clusters=3)
    inp = synth.make(w)
    idx, _ = oracle.route(inp["logits"], w.k)
    lay = oracle.layout(idx, w.E, inp["place"], w.G)
    x_disp = oracle.dispatch_rows(inp["x"], lay["disp_token"])
    sexp = oracle.slot_experts(lay["expert_off"])
    y_ref, h_ref = oracle.ffn_rows(x_disp, lay["perm_row"], sexp, inp["w_gate"], inp["w_up"],
                                   inp["w_down"], want_h=True)
    h, y = ops.moe_grouped_ffn(dev(x_disp), dev(lay["perm_row"]), dev(lay["expert_off"]), w.T,
                               w.k, dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"]))
    torch.cuda.synchronize()
    assert_close("h", host(h), h_ref, TAU["bf16"])
    assert_close("y", host(y), y_ref, TAU["bf16"])



def test_layout_workspace_is_left_zero():
    """The layout's last count block scans the counts and sets its counter in
    the workspace back to zero: the counter word reads back as zero after
    each call, and a second call on the same workspace gives the same
    layout (a stale counter would leave the bases unscanned)."""
    w = synth.with_shape(synth.workload(3), T=3000)
    inp = synth.make(w, place="contiguous", with_weights=False)
    idx, _ = oracle.route(inp["logits"], w.k)
    ref = oracle.layout(idx, w.E, inp["place"], w.G)
    out = ops.alloc_layout(w.T, w.E, w.k, w.G, "cuda")
    for _ in range(2):
        ops.moe_dispatch_layout(dev(idx), w.E, dev(inp["place"]), w.G, out=out)
        torch.cuda.synchronize()
        assert not host(out["workspace"][:256]).any()
        R = int(out["rank_off"][w.G].item())
        g = dict(rank_mask=host(out["rank_mask"]).view(np.uint32), rank_off=host(out["rank_off"]),
                 disp_token=host(out["disp_token"][:R]), expert_off=host(out["expert_off"]),
                 perm_row=host(out["perm_row"]), slot_of=host(out["slot_of"]))
        compare_exact(g, ref, ("rank_mask", "rank_off", "disp_token", "expert_off", "perm_row",
                               "slot_of"))


SCAN_CASES = [(synth.with_shape(synth.workload(3), T=T), T) for T in (3000, 8192, 8193, 9000)] + [
    (C("k3_E250", T=1001, d=64, E=250, k=3, F=64, G=10, dtype="bf16", clusters=10), 1001)]


@pytest.mark.parametrize("w,T", SCAN_CASES, ids=[f"{w.name}-T{T}" for w, T in SCAN_CASES])
@pytest.mark.parametrize("aligned", [True, False])
def test_layout_scan_paths_and_unaligned_choices(w, T, aligned):
    """The count kernel's last block scans the per-block counts in one round
    while there are at most 32 blocks of 256 tokens and E + G <= 256, in
    chunks otherwise: T = 8192 is the last size on the one-round path, and
    E + G = 260 takes the chunked one at any T. The block's choices are read
    16 bytes at a time when topk_idx is 16-byte aligned and one word at a
    time when it is not (here a view one element into a larger buffer); with
    k = 3 a block's tail is read one word at a time either way. Every case
    gives the oracle's layout bit for bit."""
    inp = synth.make(w, place="contiguous", with_weights=False)
    idx, _ = oracle.route(inp["logits"], w.k)
    ref = oracle.layout(idx, w.E, inp["place"], w.G)
    if aligned:
        d_idx = dev(idx)
    else:
        buf = torch.zeros(idx.size + 1, dtype=torch.int32, device="cuda")
        buf[1:] = dev(idx).reshape(-1)
        d_idx = buf[1:].view(idx.shape)
        assert d_idx.data_ptr() % 16 != 0
    out = ops.moe_dispatch_layout(d_idx, w.E, dev(inp["place"]), w.G)
    torch.cuda.synchronize()
    R = int(out["rank_off"][w.G].item())
    g = dict(rank_mask=host(out["rank_mask"]).view(np.uint32), rank_off=host(out["rank_off"]),
             disp_token=host(out["disp_token"][:R]), expert_off=host(out["expert_off"]),
             perm_row=host(out["perm_row"]), slot_of=host(out["slot_of"]))
    compare_exact(g, ref, ("rank_mask", "rank_off", "disp_token", "expert_off", "perm_row",
                           "slot_of"))


def test_expert_workspace_is_left_zero_and_reused():
    """The persistent expert launches claim tiles from a queue in the caller's
    workspace and leave it zero-filled: two calls in a row on one workspace
    give bit-identical h and y (a stale counter would skip tiles, leaving the
    NaN the outputs start as), and the workspace reads back as zeros. The
    shape has more tiles than two rounds of workgroups, so tiles are
    claimed from the queue."""
    rng = np.random.default_rng(41)
    T, k, E, d, F = 4096, 4, 8, 2048, 1536
    S = T * k
    counts = rng.multinomial(S, rng.dirichlet(np.ones(E)))
    eo = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = 9000
    perm = rng.integers(0, R, S).astype(np.int32)
    bf = synth.f32_to_bf16_bits
    x_disp = dev(bf(rng.standard_normal((R, d), dtype=np.float32)))
    wg = dev(bf(rng.standard_normal((E, F, d), dtype=np.float32) / np.sqrt(d)))
    wu = dev(bf(rng.standard_normal((E, F, d), dtype=np.float32) / np.sqrt(d)))
    wd = dev(bf(rng.standard_normal((E, d, F), dtype=np.float32) / np.sqrt(F)))
    ws = ops.expert_workspace("cuda")
    outs = []
    for _ in range(2):
        h = torch.full((S, F), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = torch.full((S, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        ops.moe_grouped_ffn(x_disp, dev(perm), dev(eo), T, k, wg, wu, wd, h, y, workspace=ws)
        torch.cuda.synchronize()
        assert not host(ws).any(), "workspace not left zero-filled"
        outs.append((host(h), host(y)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    slots = band_sample(eo)
    sexp = oracle.slot_experts(eo)[slots]
    y_ref, h_ref = oracle.ffn_rows(host(x_disp), perm[slots], sexp, host(wg), host(wu), host(wd),
                                   want_h=True)
    assert_close("h(bands)", outs[0][0][slots], h_ref, TAU["bf16"])
    assert_close("y(bands)", outs[0][1][slots], y_ref, TAU["bf16"])


# Segment lengths at every boundary of how a grouped launch cuts an expert's
# rows into 256-row m-tiles of whole 32-row bands split evenly over the
# expert: empty, one row, around one band, around one m-tile, two and three
# m-tiles, and nine m-tiles (where the even split leaves a one-row last tile).
SEGMENTS = [0, 1, 31, 32, 33, 255, 256, 257, 300, 511, 512, 513, 2049]


@pytest.mark.parametrize("order", ["as_listed", "reversed"])
def test_ffn_segment_boundaries(order):
    rng = np.random.default_rng(11)
    counts = SEGMENTS if order == "as_listed" else SEGMENTS[::-1]
    E, d, F, R = len(counts), 128, 192, 3000
    eo = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    S = int(eo[-1])
    perm = rng.integers(0, R, S).astype(np.int32)  # each slot reads a dispatched row
    bf = synth.f32_to_bf16_bits
    x_disp = bf(rng.standard_normal((R, d), dtype=np.float32))
    wg = bf(rng.standard_normal((E, F, d), dtype=np.float32) / np.sqrt(d))
    wu = bf(rng.standard_normal((E, F, d), dtype=np.float32) / np.sqrt(d))
    wd = bf(rng.standard_normal((E, d, F), dtype=np.float32) / np.sqrt(F))
    y_ref, h_ref = oracle.ffn_rows(x_disp, perm, oracle.slot_experts(eo), wg, wu, wd, want_h=True)
    # outputs start as NaN: a row no tile writes, or one written twice with
    # another tile's rows, fails the comparison
    h = torch.full((S, F), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full((S, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ops.moe_grouped_ffn(dev(x_disp), dev(perm), dev(eo), S, 1, dev(wg), dev(wu), dev(wd), h, y)
    torch.cuda.synchronize()
    assert_close("h", host(h), h_ref, TAU["bf16"])
    assert_close("y", host(y), y_ref, TAU["bf16"])
    # per segment as well, so a short expert's rows are not hidden by the others
    hh, yy = widen(host(h)), widen(host(y))
    for e in range(E):
        a, b = eo[e], eo[e + 1]
        if b > a:
            assert np.abs(yy[a:b] - y_ref[a:b]).max() <= TAU["bf16"] * np.abs(y_ref).max(), e
            assert np.abs(hh[a:b] - h_ref[a:b]).max() <= TAU["bf16"] * np.abs(h_ref).max(), e


# ------------------------------------------------------------------ full size

def sampled_check(w, inp, g, n_tok=48, seed=7):
    """h, y and out of a seeded sample of tokens, evaluated by the oracle."""
    rng = np.random.default_rng(seed)
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, n_tok, replace=False)]))
    idx, gates = oracle.route(inp["logits"][toks], w.k, w.n_groups, w.topk_groups)
    slots = g["slot_of"].reshape(w.T, w.k)[toks]                          # [n,k]
    y_ref, h_ref = oracle.ffn_rows(inp["x"], np.repeat(toks, w.k), idx.ravel(), inp["w_gate"],
                                   inp["w_up"], inp["w_down"], want_h=True)
    tau = TAU[w.dtype]
    assert_close("h(sample)", g["h"][slots.ravel()], h_ref, tau)
    assert_close("y(sample)", g["y"][slots.ravel()], y_ref, tau)
    n = len(toks)
    out_ref = oracle.combine(y_ref, np.arange(n * w.k, dtype=np.int32), gates, n, w.k)
    assert_close("out(sample)", g["out"][toks], out_ref, tau)


def band_sample(expert_off, seed=5, band=32):
    """One random slot in every 32-slot band of every expert's segment, plus
    each segment's last slot: every m-tile of any tiling of the segments into
    whole 32-row bands holds at least one sampled slot."""
    rng = np.random.default_rng(seed)
    picks = []
    for e in range(len(expert_off) - 1):
        a, b = int(expert_off[e]), int(expert_off[e + 1])
        for s0 in range(a, b, band):
            picks.append(rng.integers(s0, min(b, s0 + band)))
        if b > a:
            picks.append(b - 1)
    return np.unique(np.asarray(picks, np.int64))


def full_check(w, inp, g, ref_lay):
    """h and y of every slot and out of every token against the oracle."""
    x_disp = oracle.dispatch_rows(inp["x"], ref_lay["disp_token"])
    sexp = oracle.slot_experts(ref_lay["expert_off"])
    y_ref, h_ref = oracle.ffn_rows(x_disp, ref_lay["perm_row"], sexp, inp["w_gate"],
                                   inp["w_up"], inp["w_down"], want_h=True)
    tau = TAU[w.dtype]
    assert_close("h", g["h"], h_ref, tau)
    del h_ref
    assert_close("y", g["y"], y_ref, tau)
    _, gates = oracle.route(inp["logits"], w.k, w.n_groups, w.topk_groups)
    out_ref = oracle.combine(y_ref, ref_lay["slot_of"], gates, w.T, w.k)
    assert_close("out", g["out"], out_ref, tau)


def stratified_check(w, inp, g, ref_lay):
    """h and y of a band-stratified slot sample (every 32-row band of every
    expert), each slot evaluated by the oracle from its token's row; out of a
    token sample."""
    slots = band_sample(ref_lay["expert_off"])
    tok = ref_lay["disp_token"][ref_lay["perm_row"][slots]]
    sexp = oracle.slot_experts(ref_lay["expert_off"])[slots]
    y_ref, h_ref = oracle.ffn_rows(inp["x"], tok, sexp, inp["w_gate"], inp["w_up"],
                                   inp["w_down"], want_h=True)
    tau = TAU[w.dtype]
    assert_close("h(bands)", g["h"][slots], h_ref, tau)
    assert_close("y(bands)", g["y"][slots], y_ref, tau)
    sampled_check(w, inp, g)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wi", [0, 1, 2, 3, 4])
def test_full_size_parity(wi):
    w = synth.workload(wi)
    print(f"case {w.name} {w.tag()} full size", flush=True)
    inp = synth.make(w, place="contiguous")
    g = run_layer(w, DevInputs(w, inp))
    torch.cuda.empty_cache()
    idx, gates = oracle.route(inp["logits"], w.k, w.n_groups, w.topk_groups)
    ref = dict(topk_idx=idx, coact=oracle.coact(idx, w.E),
               **oracle.layout(idx, w.E, inp["place"], w.G))
    assert g["R"] == ref["R"] <= w.T * w.k
    compare_exact(g, ref)
    assert_close("gates", g["gates"], gates, TAU_GATES)
    assert np.array_equal(g["x_disp"], oracle.dispatch_rows(inp["x"], ref["disp_token"]))
    if wi <= 3:
        print(f"oracle over all {w.T * w.k} slots", flush=True)
        full_check(w, inp, g, ref)
    else:
        stratified_check(w, inp, g, ref)


@pytest.mark.timeout(300)
def test_placement_invariance_full_size():
    """Placement changes R, never the routing or the result (Zyphra page, English
    abstract: neither method alters routing decisions or expert parameters)."""
    w = synth.workload(1)
    inp = synth.make(w, place="contiguous")
    d_in = DevInputs(w, inp)
    a = run_layer(w, d_in)
    b = run_layer(w, d_in, place=dev(synth.placement(w, "colocated")))
    for key in ("topk_idx", "gates", "coact", "expert_off", "slot_of", "h", "y", "out"):
        assert np.array_equal(a[key], b[key]), key
    assert b["R"] < a["R"]


@pytest.mark.parametrize("wi,rpn", [(2, 1), (3, 8)])
def test_planned_placement_pipeline(wi, rpn):
    """Route and co-activation on the GPU, the native planner on the host
    (checked against the reference planner bit for bit), then the whole layer
    with the planned placement against the oracle; the planned placement
    sends no more rows than the index-order one."""
    from oracle import placement as OP
    w = synth.with_shape(synth.workload(wi), T=1536)
    print(f"case planned {w.name} {w.tag()} rpn={rpn}", flush=True)
    inp = synth.make(w)
    d_in = DevInputs(w, inp)
    lay = ops.Layer(w.T, w.d, w.E, w.k, w.F, w.G, torch.bfloat16, "cuda", w.n_groups,
                    w.topk_groups)
    lay.route(d_in.logits)
    lay.coact_hist()
    torch.cuda.synchronize()
    coact = host(lay.coact).astype(np.int64)
    load = np.bincount(host(lay.topk_idx).ravel(), minlength=w.E)
    plan = ops.moe_plan_placement(coact, load, w.G, rpn, 8)
    assert np.array_equal(plan, OP.plan(coact, load, w.G, rpn, 8))
    inp_p = dict(inp, place=plan)
    ref = oracle.layer(inp_p["logits"], inp_p["x"], plan, w.G, w.k, inp_p["w_gate"],
                       inp_p["w_up"], inp_p["w_down"], w.n_groups, w.topk_groups)
    g = run_layer(w, DevInputs(w, inp_p))
    assert g["R"] == ref["R"]
    compare_exact(g, ref)
    assert_close("out", g["out"], ref["out"], TAU[w.dtype])
    idx = host(lay.topk_idx)
    assert ref["R"] <= OP.dispatched_rows(idx, synth.placement(w, "contiguous"))
