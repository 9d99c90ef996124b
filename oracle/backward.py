"""TEST INFRASTRUCTURE: plain fp64 reference of the MoE layer's backward pass.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use
this. It shares no code with the library's kernels.

The pages are about training: expert parallelism runs its all-to-all in the
forward and the backward pass (Zyphra correlated expert placement page,
English abstract). They state no formulas for the backward; it is the exact
gradient of the forward this package computes, for a loss L whose gradient
with respect to the layer output is dout:

  forward, token t, choice j, expert e = idx[t, j], a = x[t]:
    u = W_gate[e] a,  v = W_up[e] a,  h = silu(u) * v,  y = W_down[e] h,
    out[t] = sum_j gates[t, j] y_tj,  gates = softmax of the chosen logits.
  backward (chain rule, written out):
    dgates[t, j] = <dout[t], y_tj>,          dy_tj = gates[t, j] dout[t]
    dh = W_down[e]^T dy,                     dW_down[e] += dy h^T
    du = dh * v * silu'(u),  dv = dh * silu(u),
      silu'(u) = s (1 + u (1 - s)),  s = 1 / (1 + e^-u)
    da = W_gate[e]^T du + W_up[e]^T dv,      dW_gate[e] += du a^T,  dW_up[e] += dv a^T
    dx[t] = sum_j da_tj
    dlogits[t, idx[t, j]] = g_j (dg_j - sum_i g_i dg_i)   (the softmax
      Jacobian over the chosen logits); the top-k selection is piecewise
      constant, so every other logit gets 0.

Matrix products (numpy matmul) serve as steps; everything is float64.
"""
from __future__ import annotations

import numpy as np


def _sig(u):
    return 1.0 / (1.0 + np.exp(-u))


def silu(u):
    return u * _sig(u)


def silu_grad(u):
    s = _sig(u)
    return s * (1.0 + u * (1.0 - s))


# ---------------------------------------------------------------- steps

def combine_bwd(dout, y, slot_of, gates):
    """-> dy [S, d] (dy[slot(t,j)] = g_tj dout[t]), dgates [T, k].

    A negative slot is a dropped choice (no expert output in the forward):
    it writes no dy row and its gate gradient is 0."""
    dout = np.asarray(dout, np.float64)
    y = np.asarray(y, np.float64)
    g = np.asarray(gates, np.float64)
    T, k = g.shape
    so = np.asarray(slot_of).reshape(T, k)
    dy = np.zeros_like(y)
    dgates = np.zeros((T, k))
    for j in range(k):
        live = so[:, j] >= 0
        s = so[live, j]
        dy[s] = g[live, j:j + 1] * dout[live]
        dgates[live, j] = (dout[live] * y[s]).sum(1)
    return dy, dgates


def swiglu_bwd(dh, u, v):
    dh, u, v = (np.asarray(a, np.float64) for a in (dh, u, v))
    return dh * v * silu_grad(u), dh * silu(u)


def down_bwd(dy, h, u, v, expert_off, w_down):
    """Per expert segment: dh = dy W_down[e] (rows), then SwiGLU backward.
    -> du, dv [S, F], dw_down [E, d, F]."""
    dy, h = np.asarray(dy, np.float64), np.asarray(h, np.float64)
    wd = np.asarray(w_down, np.float64)
    E, d, F = wd.shape
    du = np.zeros((dy.shape[0], F))
    dv = np.zeros((dy.shape[0], F))
    dwd = np.zeros((E, d, F))
    eo = np.asarray(expert_off)
    for e in range(E):
        a, b = int(eo[e]), int(eo[e + 1])
        if a == b:
            continue
        dh = dy[a:b] @ wd[e]
        du[a:b], dv[a:b] = swiglu_bwd(dh, np.asarray(u, np.float64)[a:b],
                                      np.asarray(v, np.float64)[a:b])
        dwd[e] = dy[a:b].T @ h[a:b]
    return du, dv, dwd


def gate_up_bwd(du, dv, a_rows, expert_off, w_gate, w_up):
    """a_rows [S, d]: the expert input of every slot. -> da [S, d],
    dw_gate, dw_up [E, F, d]."""
    du, dv, ar = (np.asarray(z, np.float64) for z in (du, dv, a_rows))
    wg, wu = np.asarray(w_gate, np.float64), np.asarray(w_up, np.float64)
    E, F, d = wg.shape
    da = np.zeros((du.shape[0], d))
    dwg = np.zeros((E, F, d))
    dwu = np.zeros((E, F, d))
    eo = np.asarray(expert_off)
    for e in range(E):
        a, b = int(eo[e]), int(eo[e + 1])
        if a == b:
            continue
        da[a:b] = du[a:b] @ wg[e] + dv[a:b] @ wu[e]
        dwg[e] = du[a:b].T @ ar[a:b]
        dwu[e] = dv[a:b].T @ ar[a:b]
    return da, dwg, dwu


def dispatch_bwd(da, slot_of, T, k):
    """dx[t] = sum_j da[slot(t, j)] over the choices with a slot (a negative
    slot is a dropped choice and adds nothing)."""
    da = np.asarray(da, np.float64)
    so = np.asarray(slot_of).reshape(T, k)
    dx = np.zeros((T, da.shape[1]))
    for j in range(k):
        live = so[:, j] >= 0
        dx[live] += da[so[live, j]]
    return dx


def route_bwd(gates, dgates, topk_idx, E):
    g = np.asarray(gates, np.float64)
    dg = np.asarray(dgates, np.float64)
    idx = np.asarray(topk_idx)
    T, k = g.shape
    dl = np.zeros((T, E))
    inner = (g * dg).sum(1, keepdims=True)
    np.put_along_axis(dl, idx.astype(np.int64), g * (dg - inner), axis=1)
    return dl


# ---------------------------------------------------------------- whole layer

def forward64(logits, x, w_gate, w_up, w_down, k):
    """fp64 forward of the layer (plain top-k routing, ties to the lower
    expert index) in token order; used to check the backward by finite
    differences. -> out [T, d] and every intermediate."""
    L = np.asarray(logits, np.float64)
    x = np.asarray(x, np.float64)
    wg, wu, wd = (np.asarray(w, np.float64) for w in (w_gate, w_up, w_down))
    T, E = L.shape
    idx = np.argsort(-L, axis=1, kind="stable")[:, :k]
    z = np.take_along_axis(L, idx, axis=1)
    g = np.exp(z - z.max(1, keepdims=True))
    g /= g.sum(1, keepdims=True)
    out = np.zeros_like(x)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            u, v = wg[e] @ x[t], wu[e] @ x[t]
            out[t] += g[t, j] * (wd[e] @ (silu(u) * v))
    return out, idx, g


def layer_backward(topk_idx, gates, x, w_gate, w_up, w_down, dout):
    """Gradients of <dout, out> for a given routing (topk_idx, gates), in
    token-choice order (slot = t * k + j). -> dict of dx, dlogits (needs E:
    taken from the weights), dgates, dw_gate, dw_up, dw_down and the
    intermediates."""
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    wg = np.asarray(w_gate, np.float64)
    E = wg.shape[0]
    x = np.asarray(x, np.float64)
    # slots in expert-grouped order (experts ascending, then t, then j)
    t_of, j_of = np.divmod(np.arange(T * k), k)
    e_of = idx.reshape(-1)
    order = np.lexsort((j_of, t_of, e_of))
    slot_of = np.empty(T * k, np.int64)
    slot_of[order] = np.arange(T * k)
    expert_off = np.concatenate([[0], np.cumsum(np.bincount(e_of, minlength=E))])
    a_rows = x[t_of[order]]
    wu, wd = np.asarray(w_up, np.float64), np.asarray(w_down, np.float64)
    u = np.empty((T * k, wg.shape[1]))
    v = np.empty_like(u)
    y = np.empty((T * k, x.shape[1]))
    for e in range(E):
        a, b = int(expert_off[e]), int(expert_off[e + 1])
        u[a:b] = a_rows[a:b] @ wg[e].T
        v[a:b] = a_rows[a:b] @ wu[e].T
        y[a:b] = (silu(u[a:b]) * v[a:b]) @ wd[e].T
    h = silu(u) * v
    dy, dgates = combine_bwd(dout, y, slot_of, gates)
    du, dv, dwd = down_bwd(dy, h, u, v, expert_off, wd)
    da, dwg, dwu = gate_up_bwd(du, dv, a_rows, expert_off, wg, wu)
    dx = dispatch_bwd(da, slot_of, T, k)
    dl = route_bwd(gates, dgates, idx, E)
    return dict(dx=dx, dlogits=dl, dgates=dgates, dw_gate=dwg, dw_up=dwu, dw_down=dwd,
                dy=dy, du=du, dv=dv, da=da, u=u, v=v, h=h, y=y, slot_of=slot_of,
                expert_off=expert_off)
