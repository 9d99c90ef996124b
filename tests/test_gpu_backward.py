"""GPU parity of the backward pass against the fp64 reference backward.

Per step on seeded random inputs (ragged expert segments with empty and
single-slot experts, output widths that leave partial tiles, bf16 and fp32),
then the whole layer (forward with saved pre-activations, then every
backward step) against oracle.backward.layer_backward, and at the full
T=8192, d=4096, E=128, k=8, F=1536 size on sampled experts and tokens that the
reference evaluates on its own. Tolerance: max|gpu - ref| <= tau * max|ref|
per tensor, tau = 1e-4 (fp32) and 2e-2 (bf16) as in the forward tests. The
fp32 weight gradients of the step and segment tests, whose inputs the GPU
reads exactly, are held to 1e-4 per expert; in the whole-layer tests they are
computed from bf16-rounded intermediates (dy, du, dv, h), so the bf16
tolerance bounds them there.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as OB
from routing_dispatch_expert_top_amd import ops, synth
from tests.gpu_helpers import TAU, assert_close, dev, host, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()


def _store(a, dtype):
    a = np.asarray(a, np.float32)
    return synth.f32_to_bf16_bits(a) if dtype == "bf16" else a


def _w(a):
    return widen(a) if a.dtype in (np.uint16, np.float32) else np.asarray(a, np.float64)


def per_expert_close(name, got, ref, eo):
    """fp32 weight gradients whose inputs are exact (bf16 or fp32 values the
    GPU reads as they are): fp32 accumulation error only, so each expert is
    held to the fp32 tolerance against its own largest reference entry, and
    an expert without slots must be exactly zero."""
    for e in range(len(eo) - 1):
        if eo[e + 1] == eo[e]:
            assert (got[e] == 0).all(), f"{name}[{e}] of an empty expert is not zero"
        else:
            assert_close(f"{name}[{e}]", got[e], ref[e], TAU["f32"])


def _ragged_offsets(E, S, rng):
    """Segment lengths with empty, single-slot and long experts."""
    cuts = np.sort(rng.integers(0, S + 1, size=E - 1))
    lens = np.diff(np.concatenate([[0], cuts, [S]]))
    if E >= 4:
        lens[1] += lens[0]
        lens[0] = 0                      # an empty expert
        lens[2] += lens[3] - 1
        lens[3] = 1                      # a single slot
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


STEP_CASES = [  # T, k, E, d, F, dtype, seed
    (300, 2, 6, 192, 320, "bf16", 0),
    (129, 4, 8, 256, 128, "f32", 1),
    (700, 3, 5, 128, 192, "bf16", 2),
    (64, 1, 4, 64, 64, "bf16", 3),
]


# Rows of several 1 KiB blocks for the combine kernels, which hold a row of at
# most 8 KiB in registers and walk longer rows block by block: 5 blocks with
# a partial last one (bf16 d 2368), 9 with a partial last one (bf16 d 4160,
# fp32 d 2112), and k values with and without a k-specific kernel.
LONG_ROW_CASES = [
    (80, 6, 12, 2368, 64, "bf16", 5),
    (96, 8, 16, 4160, 64, "bf16", 6),
    (40, 3, 6, 2112, 64, "f32", 7),
]


@pytest.mark.parametrize("T,k,E,d,F,dtype,seed", STEP_CASES + LONG_ROW_CASES)
def test_combine_and_route_bwd(T, k, E, d, F, dtype, seed):
    rng = np.random.default_rng(seed)
    S = T * k
    dout = _store(rng.standard_normal((T, d)), dtype)
    y = _store(rng.standard_normal((S, d)), dtype)
    slot_of = rng.permutation(S).astype(np.int32)
    z = rng.standard_normal((T, k))
    gates = (np.exp(z) / np.exp(z).sum(1, keepdims=True)).astype(np.float32)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    dy, dg = ops.moe_combine_bwd(dev(dout), dev(y), dev(slot_of), dev(gates), T, k)
    dl = ops.moe_route_bwd(dev(gates), dg, dev(idx), E)
    torch.cuda.synchronize()
    ref_dy, ref_dg = OB.combine_bwd(_w(dout), _w(y), slot_of, gates)
    assert_close("dy", host(dy), ref_dy, TAU[dtype])
    assert_close("dgates", host(dg), ref_dg, 1e-4)
    # routing backward on the GPU's dgates (fp32) against the reference on the same values
    ref_dl = OB.route_bwd(gates, host(dg), idx, E)
    assert_close("dlogits", host(dl), ref_dl, 1e-4)
    da = _store(rng.standard_normal((S, d)), dtype)
    dx = ops.moe_dispatch_bwd(dev(da), dev(slot_of), T, k)
    torch.cuda.synchronize()
    assert_close("dx", host(dx), OB.dispatch_bwd(_w(da), slot_of, T, k), TAU[dtype])


@pytest.mark.parametrize("T,k,E,d,F,dtype,seed", LONG_ROW_CASES + [(40, 8, 8, 4096, 64, "bf16", 8)])
def test_combine_long_rows_with_dropped_choices(T, k, E, d, F, dtype, seed):
    """The forward combine on rows of several 1 KiB blocks (held in registers
    up to 8 KiB, exactly 8 blocks included; block by block beyond), with about
    a tenth of the choices dropped (negative slot): a dropped choice is the
    same as one pointing at an all-zero row."""
    rng = np.random.default_rng(seed)
    S = T * k
    y = _store(rng.standard_normal((S, d)), dtype)
    slot_of = rng.permutation(S).astype(np.int32)
    drop = rng.random(S) < 0.1
    drop[:k] = True                                       # token 0: every choice dropped
    gates = rng.random((T, k)).astype(np.float32)
    out = ops.moe_combine(dev(y), dev(np.where(drop, -1, slot_of).astype(np.int32)), dev(gates),
                          T, k)
    torch.cuda.synchronize()
    y_z = np.vstack([_w(y), np.zeros((1, d))])
    ref = oracle.combine(y_z, np.where(drop, S, slot_of).astype(np.int32),
                         gates.astype(np.float64), T, k)
    got = host(out)
    assert not got[0].any()
    assert_close("out", got, ref, TAU[dtype])
    # the combine backward on the same layout: live slots get g dout, dropped
    # choices get dgates 0 (the zero row's dot product)
    dout = _store(rng.standard_normal((T, d)), dtype)
    so_d = np.where(drop, -1, slot_of).astype(np.int32)
    dy, dg = ops.moe_combine_bwd(dev(dout), dev(y), dev(so_d), dev(gates), T, k)
    torch.cuda.synchronize()
    g_z = np.where(drop.reshape(T, k), 0.0, gates.astype(np.float64))
    ref_dy, ref_dg = OB.combine_bwd(_w(dout), y_z, np.where(drop, S, slot_of).astype(np.int32), g_z)
    live = slot_of[~drop]
    assert_close("dy", host(dy)[live], ref_dy[live], TAU[dtype])
    assert_close("dgates", host(dg), ref_dg, 1e-4)
    assert not host(dg)[0].any()


@pytest.mark.parametrize("T,k,E,d,F,dtype,seed", STEP_CASES)
def test_expert_bwd_steps(T, k, E, d, F, dtype, seed):
    rng = np.random.default_rng(seed + 100)
    S = T * k
    eo = _ragged_offsets(E, S, rng)
    dy = _store(rng.standard_normal((S, d)), dtype)
    h = _store(rng.standard_normal((S, F)), dtype)
    uv = _store(rng.standard_normal((S, 2 * F)) * 2, dtype)
    wd = _store(rng.standard_normal((E, d, F)) / np.sqrt(F), dtype)
    duv, dwd = ops.moe_expert_down_bwd(dev(dy), dev(h), dev(uv), dev(eo), T, k, dev(wd))
    torch.cuda.synchronize()
    u, v = _w(uv)[:, :F], _w(uv)[:, F:]
    rdu, rdv, rdwd = OB.down_bwd(_w(dy), _w(h), u, v, eo, _w(wd))
    g_duv = host(duv)
    assert_close("du", g_duv[:, :F], rdu, TAU[dtype])
    assert_close("dv", g_duv[:, F:], rdv, TAU[dtype])
    per_expert_close("dw_down", host(dwd), rdwd, eo)

    R = S + 5
    x_disp = _store(rng.standard_normal((R, d)), dtype)
    perm_row = rng.integers(0, R, size=S).astype(np.int32)
    duv_in = _store(rng.standard_normal((S, 2 * F)), dtype)
    wg = _store(rng.standard_normal((E, F, d)) / np.sqrt(d), dtype)
    wu = _store(rng.standard_normal((E, F, d)) / np.sqrt(d), dtype)
    da, dwg, dwu = ops.moe_expert_gate_up_bwd(dev(duv_in), dev(x_disp), dev(perm_row), dev(eo),
                                              T, k, dev(wg), dev(wu))
    torch.cuda.synchronize()
    rda, rdwg, rdwu = OB.gate_up_bwd(_w(duv_in)[:, :F], _w(duv_in)[:, F:], _w(x_disp)[perm_row],
                                     eo, _w(wg), _w(wu))
    assert_close("da", host(da), rda, TAU[dtype])
    per_expert_close("dw_gate", host(dwg), rdwg, eo)
    per_expert_close("dw_up", host(dwu), rdwu, eo)



# Expert segment lengths at every boundary of the grouped launches' tiling
# (32-row bands, 256-row m-tiles split evenly over an expert, 64-slot K tiles
# of the weight gradients): empty, one slot, around one band, around one
# m-tile, two and three m-tiles, nine m-tiles.
SEGMENTS = [0, 1, 31, 32, 33, 63, 64, 65, 255, 256, 257, 300, 511, 512, 513, 2049]


def test_expert_bwd_segment_boundaries():
    rng = np.random.default_rng(23)
    E, d, F = len(SEGMENTS), 128, 192
    eo = np.concatenate([[0], np.cumsum(SEGMENTS)]).astype(np.int32)
    S = int(eo[-1])
    bf = lambda a: _store(a, "bf16")
    dy, h = bf(rng.standard_normal((S, d))), bf(rng.standard_normal((S, F)))
    uv = bf(rng.standard_normal((S, 2 * F)) * 2)
    wd = bf(rng.standard_normal((E, d, F)) / np.sqrt(F))
    nan = float("nan")
    # outputs start as NaN: a row or gradient tile no launch writes fails
    duv = torch.full((S, 2 * F), nan, dtype=torch.bfloat16, device="cuda")
    dwd = torch.full((E, d, F), nan, dtype=torch.float32, device="cuda")
    ops.moe_expert_down_bwd(dev(dy), dev(h), dev(uv), dev(eo), S, 1, dev(wd), duv, dwd)
    torch.cuda.synchronize()
    u, v = _w(uv)[:, :F], _w(uv)[:, F:]
    rdu, rdv, rdwd = OB.down_bwd(_w(dy), _w(h), u, v, eo, _w(wd))
    g_duv = host(duv)
    assert_close("du", g_duv[:, :F], rdu, TAU["bf16"])
    assert_close("dv", g_duv[:, F:], rdv, TAU["bf16"])
    per_expert_close("dw_down", host(dwd), rdwd, eo)

    R = 3000
    x_disp = bf(rng.standard_normal((R, d)))
    perm_row = rng.integers(0, R, size=S).astype(np.int32)
    duv_in = bf(rng.standard_normal((S, 2 * F)))
    wg = bf(rng.standard_normal((E, F, d)) / np.sqrt(d))
    wu = bf(rng.standard_normal((E, F, d)) / np.sqrt(d))
    da = torch.full((S, d), nan, dtype=torch.bfloat16, device="cuda")
    dwg = torch.full((E, F, d), nan, dtype=torch.float32, device="cuda")
    dwu = torch.full((E, F, d), nan, dtype=torch.float32, device="cuda")
    ops.moe_expert_gate_up_bwd(dev(duv_in), dev(x_disp), dev(perm_row), dev(eo), S, 1, dev(wg),
                               dev(wu), da, dwg, dwu)
    torch.cuda.synchronize()
    rda, rdwg, rdwu = OB.gate_up_bwd(_w(duv_in)[:, :F], _w(duv_in)[:, F:], _w(x_disp)[perm_row],
                                     eo, _w(wg), _w(wu))
    assert_close("da", host(da), rda, TAU["bf16"])
    per_expert_close("dw_gate", host(dwg), rdwg, eo)
    per_expert_close("dw_up", host(dwu), rdwu, eo)
    # da per expert as well, so a short segment's rows are not hidden by the others
    for e in range(E):
        a, b = eo[e], eo[e + 1]
        if b > a:
            assert_close(f"da[{e}]", host(da)[a:b], rda[a:b], TAU["bf16"])

def test_expert_bwd_workspace_reused():
    """The weight-gradient launches are persistent: their tile queue lives in
    the backward workspace, is cleared before each launch and left zero.
    Two rounds of both expert backward calls through one workspace, outputs
    NaN-filled before each call (a tile a stale queue skipped stays NaN),
    give the same bits, and the first matches the reference. E = 13 leaves
    unused positions in the expert walk."""
    rng = np.random.default_rng(31)
    T, k, E, d, F = 500, 3, 13, 128, 192
    S = T * k
    eo = _ragged_offsets(E, S, rng)
    bf = lambda a: _store(a, "bf16")
    dy, h = bf(rng.standard_normal((S, d))), bf(rng.standard_normal((S, F)))
    uv = bf(rng.standard_normal((S, 2 * F)) * 2)
    wd = bf(rng.standard_normal((E, d, F)) / np.sqrt(F))
    R = S + 7
    x_disp = bf(rng.standard_normal((R, d)))
    perm_row = rng.integers(0, R, size=S).astype(np.int32)
    wg = bf(rng.standard_normal((E, F, d)) / np.sqrt(d))
    wu = bf(rng.standard_normal((E, F, d)) / np.sqrt(d))
    ws = ops.bwd_workspace(T, E, k, d, F, "cuda")
    nan = float("nan")
    outs = []
    for _ in range(2):
        duv = torch.full((S, 2 * F), nan, dtype=torch.bfloat16, device="cuda")
        dwd = torch.full((E, d, F), nan, dtype=torch.float32, device="cuda")
        ops.moe_expert_down_bwd(dev(dy), dev(h), dev(uv), dev(eo), T, k, dev(wd), duv, dwd,
                                workspace=ws)
        da = torch.full((S, d), nan, dtype=torch.bfloat16, device="cuda")
        dwg = torch.full((E, F, d), nan, dtype=torch.float32, device="cuda")
        dwu = torch.full((E, F, d), nan, dtype=torch.float32, device="cuda")
        ops.moe_expert_gate_up_bwd(duv, dev(x_disp), dev(perm_row), dev(eo), T, k, dev(wg),
                                   dev(wu), da, dwg, dwu, workspace=ws)
        torch.cuda.synchronize()
        outs.append([host(t) for t in (duv, dwd, da, dwg, dwu)])
    for name, a, b in zip(("duv", "dw_down", "da", "dw_gate", "dw_up"), outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
    u, v = _w(uv)[:, :F], _w(uv)[:, F:]
    _, _, rdwd = OB.down_bwd(_w(dy), _w(h), u, v, eo, _w(wd))
    per_expert_close("dw_down", outs[0][1], rdwd, eo)
    duv_g = outs[0][0]
    _, rdwg, rdwu = OB.gate_up_bwd(_w(duv_g)[:, :F], _w(duv_g)[:, F:], _w(x_disp)[perm_row], eo,
                                   _w(wg), _w(wu))
    per_expert_close("dw_gate", outs[0][3], rdwg, eo)
    per_expert_close("dw_up", outs[0][4], rdwu, eo)


SAVE_CASES = [
    synth.custom(name="bf16_save_ragged", T=700, d=256, E=6, k=2, F=320, G=2, dtype="bf16",
                 clusters=2),
    synth.custom(name="bf16_save_long_k", T=1500, d=1024, E=4, k=2, F=192, G=2, dtype="bf16",
                 clusters=2),
]


@pytest.mark.parametrize("w", SAVE_CASES, ids=[w.name for w in SAVE_CASES])
def test_gate_up_save_outputs(w):
    """The training gate/up (persistent launch, h then u then v staged and
    stored in turn) against the plain forward gate/up (h bit for bit) and
    against the fp64 reference's u, v and h in slot order. F = 320 leaves a
    half-filled column tile; d = 1024 runs 16 K slices; experts of 214 to
    764 slots leave ragged m-tiles."""
    print(f"case gate_up_save {w.name} {w.tag()}", flush=True)
    inp = synth.make(w)
    lay = ops.Layer(w.T, w.d, w.E, w.k, w.F, w.G, torch.bfloat16, "cuda", w.n_groups,
                    w.topk_groups)
    lay.route(dev(inp["logits"]))
    lay.dispatch(dev(inp["x"]), dev(inp["place"]))
    L = lay.lay
    wg, wu = dev(inp["w_gate"]), dev(inp["w_up"])
    h_plain = ops.moe_expert_gate_up(L["x_disp"], L["perm_row"], L["expert_off"], w.T, w.k, wg, wu)
    h, uv = ops.moe_expert_gate_up_save(L["x_disp"], L["perm_row"], L["expert_off"], w.T, w.k,
                                        wg, wu)
    torch.cuda.synchronize()
    assert torch.equal(h, h_plain)
    idx, gates = oracle.route(inp["logits"], w.k)
    assert np.array_equal(host(lay.topk_idx), idx)
    ref = OB.layer_backward(idx, gates, synth.to_f64(inp["x"], "bf16"),
                            synth.to_f64(inp["w_gate"], "bf16"), synth.to_f64(inp["w_up"], "bf16"),
                            synth.to_f64(inp["w_down"], "bf16"), np.zeros((w.T, w.d)))
    g_uv = host(uv)
    assert_close("u", g_uv[:, :w.F], ref["u"], TAU["bf16"])
    assert_close("v", g_uv[:, w.F:], ref["v"], TAU["bf16"])
    assert_close("h", host(h), ref["h"], TAU["bf16"])


def _gpu_train_step(w, inp, dout, place):
    """Forward (saving u, v) and every backward step on the GPU."""
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    lay = ops.Layer(w.T, w.d, w.E, w.k, w.F, w.G, dt, "cuda", w.n_groups, w.topk_groups)
    x = dev(inp["x"])
    wg, wu, wd = dev(inp["w_gate"]), dev(inp["w_up"]), dev(inp["w_down"])
    lay.route(dev(inp["logits"]))
    lay.dispatch(x, dev(place))
    L = lay.lay
    h, uv = ops.moe_expert_gate_up_save(L["x_disp"], L["perm_row"], L["expert_off"], w.T, w.k,
                                        wg, wu)
    y = ops.moe_expert_down(h, L["expert_off"], w.T, w.k, wd)
    dy, dgates = ops.moe_combine_bwd(dev(dout), y, L["slot_of"], lay.gates, w.T, w.k)
    duv, dwd = ops.moe_expert_down_bwd(dy, h, uv, L["expert_off"], w.T, w.k, wd)
    da, dwg, dwu = ops.moe_expert_gate_up_bwd(duv, L["x_disp"], L["perm_row"], L["expert_off"],
                                              w.T, w.k, wg, wu)
    dx = ops.moe_dispatch_bwd(da, L["slot_of"], w.T, w.k)
    dl = ops.moe_route_bwd(lay.gates, dgates, lay.topk_idx, w.E)
    torch.cuda.synchronize()
    return dict(topk_idx=lay.topk_idx, gates=lay.gates, dx=dx, dlogits=dl, dgates=dgates,
                dw_gate=dwg, dw_up=dwu, dw_down=dwd, expert_off=L["expert_off"])


LAYER_CASES = [
    synth.workload(0),
    synth.custom(name="bf16_bwd", T=400, d=192, E=8, k=3, F=128, G=4, dtype="bf16", clusters=4,
                 boost=2.0),
    synth.custom(name="bf16_bwd_grouped", T=257, d=128, E=16, k=4, F=192, G=4, dtype="bf16",
                 clusters=4, n_groups=4, topk_groups=2),
]


@pytest.mark.parametrize("w", LAYER_CASES, ids=[w.name for w in LAYER_CASES])
def test_layer_backward(w):
    print(f"case backward {w.name} {w.tag()}", flush=True)
    inp = synth.make(w)
    dout = _store(np.random.default_rng(9).standard_normal((w.T, w.d)), w.dtype)
    g = _gpu_train_step(w, inp, dout, inp["place"])
    idx, gates = oracle.route(inp["logits"], w.k, w.n_groups, w.topk_groups)
    assert np.array_equal(host(g["topk_idx"]), idx)
    ref = OB.layer_backward(idx, gates, synth.to_f64(inp["x"], w.dtype),
                            synth.to_f64(inp["w_gate"], w.dtype), synth.to_f64(inp["w_up"], w.dtype),
                            synth.to_f64(inp["w_down"], w.dtype), _w(dout))
    tau = TAU[w.dtype]
    for key in ("dx", "dgates", "dw_gate", "dw_up", "dw_down"):
        assert_close(key, host(g[key]), ref[key], tau)
    # dlogits: the softmax Jacobian subtracts the gate-weighted mean of dgates;
    # checked against the reference Jacobian applied to the reference dgates
    assert_close("dlogits", host(g["dlogits"]), ref["dlogits"], tau)


@pytest.mark.timeout(900)
def test_full_size_backward_sampled():
    """T=8192, d=4096, E=128, k=8, F=1536, bf16: weight gradients of two
    experts (a busy and a light one) and dx / dlogits of sampled tokens, each
    evaluated by the reference from the inputs alone."""
    w = synth.workload(3)
    print(f"case backward full {w.tag()}", flush=True)
    inp = synth.make(w)
    dout = _store(np.random.default_rng(9).standard_normal((w.T, w.d)), "bf16")
    g = _gpu_train_step(w, inp, dout, inp["place"])
    idx, gates = oracle.route(inp["logits"], w.k)
    assert np.array_equal(host(g["topk_idx"]), idx)
    x64 = synth.to_f64(inp["x"], "bf16")
    counts = np.bincount(idx.ravel(), minlength=w.E)
    busy, light = int(counts.argmax()), int(np.argsort(counts)[w.E // 4])
    dout64 = _w(dout)
    for e in (busy, light):
        t_of, j_of = np.nonzero(idx == e)
        wg = synth.to_f64(inp["w_gate"][e], "bf16")
        wu = synth.to_f64(inp["w_up"][e], "bf16")
        wd = synth.to_f64(inp["w_down"][e], "bf16")
        a = x64[t_of]
        u, v = a @ wg.T, a @ wu.T
        h = OB.silu(u) * v
        dy = np.asarray(gates, np.float64)[t_of, j_of][:, None] * dout64[t_of]
        du, dv = OB.swiglu_bwd(dy @ wd, u, v)
        for key, ref in (("dw_down", dy.T @ h), ("dw_gate", du.T @ a), ("dw_up", dv.T @ a)):
            got = g[key][e].cpu().numpy()
            assert_close(f"{key}[{e}]", got, ref, TAU["bf16"])
    rng = np.random.default_rng(4)
    toks = rng.choice(w.T, size=12, replace=False)
    dx = host(g["dx"][torch.as_tensor(toks, device="cuda")])
    dl = g["dlogits"][torch.as_tensor(toks, device="cuda")].cpu().numpy()
    ref_dx = np.zeros((len(toks), w.d))
    ref_dl = np.zeros((len(toks), w.E))
    for n, t in enumerate(toks):
        dg = np.zeros(w.k)
        gt = np.asarray(gates, np.float64)[t]
        for j in range(w.k):
            e = idx[t, j]
            wg = synth.to_f64(inp["w_gate"][e], "bf16")
            wu = synth.to_f64(inp["w_up"][e], "bf16")
            wd = synth.to_f64(inp["w_down"][e], "bf16")
            u, v = wg @ x64[t], wu @ x64[t]
            y = wd @ (OB.silu(u) * v)
            dg[j] = dout64[t] @ y
            du, dv = OB.swiglu_bwd((gt[j] * dout64[t]) @ wd, u, v)
            ref_dx[n] += du @ wg + dv @ wu
        ref_dl[n] = OB.route_bwd(gt[None], dg[None], idx[t][None], w.E)[0]
    assert_close("dx[sampled]", dx, ref_dx, TAU["bf16"])
    assert_close("dlogits[sampled]", dl, ref_dl, TAU["bf16"])
