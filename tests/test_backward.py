"""Pins of the fp64 reference backward (oracle/backward.py).

The backward is the exact gradient of the layer's forward for a loss with
gradient dout at the output; it is pinned by central finite differences of
an independent fp64 forward (every input: activations, all three weight
stacks and the router logits), by agreement of its forward recompute with the
C oracle's layer, and by invariants of the softmax Jacobian.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as B


def _tiny(seed, T=6, d=8, E=5, k=2, F=4):
    rng = np.random.default_rng(seed)
    return dict(logits=rng.standard_normal((T, E)), x=rng.standard_normal((T, d)),
                w_gate=rng.standard_normal((E, F, d)) * 0.5, w_up=rng.standard_normal((E, F, d)) * 0.5,
                w_down=rng.standard_normal((E, d, F)) * 0.5, dout=rng.standard_normal((T, d)), k=k)


def _loss(p):
    out, _, _ = B.forward64(p["logits"], p["x"], p["w_gate"], p["w_up"], p["w_down"], p["k"])
    return float((out * p["dout"]).sum())


@pytest.mark.parametrize("seed,k", [(0, 2), (1, 3), (2, 1)])
def test_gradients_match_finite_differences(seed, k):
    p = _tiny(seed, k=k)
    out, idx, g = B.forward64(p["logits"], p["x"], p["w_gate"], p["w_up"], p["w_down"], k)
    gr = B.layer_backward(idx, g, p["x"], p["w_gate"], p["w_up"], p["w_down"], p["dout"])
    eps = 1e-6
    for name, key in [("x", "dx"), ("w_gate", "dw_gate"), ("w_up", "dw_up"),
                      ("w_down", "dw_down"), ("logits", "dlogits")]:
        a = p[name]
        num = np.zeros_like(a)
        for i in np.ndindex(a.shape):
            old = a[i]
            a[i] = old + eps
            lp = _loss(p)
            a[i] = old - eps
            lm = _loss(p)
            a[i] = old
            num[i] = (lp - lm) / (2 * eps)
        err = np.abs(num - gr[key]).max()
        assert err <= 1e-6 * max(1.0, np.abs(num).max()), f"{name}: {err}"


def test_forward_recompute_matches_c_oracle():
    rng = np.random.default_rng(5)
    T, d, E, k, F, G = 40, 16, 8, 3, 12, 4
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = (rng.standard_normal((E, F, d)) * 0.3).astype(np.float32)
    wu = (rng.standard_normal((E, F, d)) * 0.3).astype(np.float32)
    wd = (rng.standard_normal((E, d, F)) * 0.3).astype(np.float32)
    ref = oracle.layer(logits, x, np.arange(E, dtype=np.int32) % G, G, k, wg, wu, wd)
    gr = B.layer_backward(ref["topk_idx"], ref["gates"], x, wg, wu, wd, np.zeros((T, d)))
    so = gr["slot_of"].reshape(T, k)
    out = sum(np.asarray(ref["gates"], np.float64)[:, j:j + 1] * gr["y"][so[:, j]] for j in range(k))
    assert np.abs(out - ref["out"]).max() <= 1e-12 * max(1.0, np.abs(ref["out"]).max())
    assert np.array_equal(gr["slot_of"], ref["slot_of"])


def test_softmax_jacobian_invariants():
    rng = np.random.default_rng(7)
    T, E, k = 50, 12, 4
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k]
    z = rng.standard_normal((T, k))
    g = np.exp(z) / np.exp(z).sum(1, keepdims=True)
    dg = rng.standard_normal((T, k))
    dl = B.route_bwd(g, dg, idx, E)
    assert np.abs(dl.sum(1)).max() < 1e-12          # rows of the Jacobian sum to zero
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, idx, True, axis=1)
    assert (dl[~mask] == 0).all()
    # k = 1: the single gate is 1 whatever the logit
    assert (B.route_bwd(np.ones((T, 1)), dg[:, :1], idx[:, :1], E) == 0).all()
    # dgates along the gates direction changes nothing
    assert np.abs(B.route_bwd(g, dg + 3.0, idx, E) - dl).max() < 1e-12


def test_unused_expert_gets_zero_weight_gradient():
    p = _tiny(3, T=4, E=6, k=2)
    p["logits"][:, 5] = -50.0
    out, idx, g = B.forward64(p["logits"], p["x"], p["w_gate"], p["w_up"], p["w_down"], 2)
    assert not (idx == 5).any()
    gr = B.layer_backward(idx, g, p["x"], p["w_gate"], p["w_up"], p["w_down"], p["dout"])
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert (gr[key][5] == 0).all()
    assert (gr["dlogits"][:, 5] == 0).all()


def test_silu_grad_closed_forms():
    assert B.silu_grad(np.array([0.0]))[0] == 0.5
    u = np.array([-30.0, 30.0])
    assert np.allclose(B.silu_grad(u), [0.0, 1.0], atol=1e-10)


def test_dropped_choices_are_zero_rows():
    """A dropped choice (negative slot) acts as an expert output of zero with
    weight zero: combine_bwd and dispatch_bwd on it equal the same calls with
    the choice pointed at an extra all-zero row, which is then removed."""
    rng = np.random.default_rng(8)
    T, k, d = 30, 4, 6
    S = T * k
    so = rng.permutation(S).astype(np.int32)
    drop = rng.random(S) < 0.25
    drop[:k] = True
    so_d = np.where(drop, -1, so).astype(np.int32)
    so_z = np.where(drop, S, so).astype(np.int32)        # the extra zero row
    dout = rng.standard_normal((T, d))
    y = rng.standard_normal((S, d))
    gates = rng.random((T, k))
    y_z = np.vstack([y, np.zeros((1, d))])
    dy, dg = B.combine_bwd(dout, y, so_d, gates)
    g_z = np.where(drop.reshape(T, k), 0.0, gates)
    dy_z, dg_z = B.combine_bwd(dout, y_z, so_z, g_z)
    assert np.array_equal(dy, dy_z[:S]) and np.array_equal(dg, dg_z)
    assert not dg[0].any()
    da = rng.standard_normal((S, d))
    dx = B.dispatch_bwd(da, so_d, T, k)
    dx_z = B.dispatch_bwd(np.vstack([da, np.zeros((1, d))]), so_z, T, k)
    assert np.array_equal(dx, dx_z) and not dx[0].any()
