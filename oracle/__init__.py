"""fp64 CPU reference of the MoE-layer hot path (TEST INFRASTRUCTURE).

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package. It wraps ``oracle.c`` (plain C, built with
gcc into ``liboracle.so``) through ctypes and composes its step functions into
a whole layer. Nothing here imports or calls the HIP library.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
_lib = None


def compile_c(src: str, out: str) -> str:
    """gcc build of a copy of oracle.c (OpenMP, no fast-math, no FP contraction)."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off",
                           "-fno-fast-math", "-Wall", "-Wextra", "-shared", "-fPIC",
                           src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_c(_SRC, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(C.CDLL(_LIB))
    return _lib


def _bind(L):
    p = C.c_void_p
    i = C.c_int
    L.orc_route.argtypes = [p, i, i, i, i, i, p, p]
    L.orc_coact.argtypes = [p, i, i, i, p]
    L.orc_layout.argtypes = [p, i, i, i, p, i, p, p, p, p, p, p]
    L.orc_dispatch_rows.argtypes = [p, i, i, i, p, i, p]
    L.orc_ffn_rows.argtypes = [p, i, i, i, i, p, p, i, p, p, p, p, p]
    L.orc_combine.argtypes = [p, i, p, p, i, i, i, p]
    L.orc_threads.argtypes = []
    L.orc_threads.restype = C.c_int
    for f in (L.orc_route, L.orc_coact, L.orc_layout, L.orc_dispatch_rows,
              L.orc_ffn_rows, L.orc_combine):
        f.restype = C.c_int
    return L


class use_library:
    """Context manager: route every wrapper call to another build of oracle.c
    (the pin suite uses it to show that planted mistakes are caught)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = _bind(C.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"activations/weights must be float32 or bf16 bits (uint16), got {a.dtype}")


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_threads())


# ---------------------------------------------------------------- step wrappers

def route(logits, k, n_groups=1, topk_groups=1):
    """-> topk_idx [T,k] int32, gates [T,k] float64."""
    L = _c(logits, np.float32)
    T, E = L.shape
    idx = np.empty((T, k), np.int32)
    g = np.empty((T, k), np.float64)
    _check(lib().orc_route(_p(L), T, E, k, n_groups, topk_groups, _p(idx), _p(g)), "route")
    return idx, g


def coact(topk_idx, E):
    """-> coact [E,E] int64 (fresh count)."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    out = np.empty((E, E), np.int64)
    _check(lib().orc_coact(_p(idx), T, E, k, _p(out)), "coact")
    return out


def layout(topk_idx, E, place, G):
    """-> dict(rank_mask, rank_off, disp_token, expert_off, perm_row, slot_of, R)."""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    pl = _c(place, np.int32)
    rm = np.empty(T, np.uint32)
    ro = np.empty(G + 1, np.int32)
    dtok = np.empty(T * k, np.int32)
    eo = np.empty(E + 1, np.int32)
    pr = np.empty(T * k, np.int32)
    so = np.empty(T * k, np.int32)
    _check(lib().orc_layout(_p(idx), T, E, k, _p(pl), G, _p(rm), _p(ro), _p(dtok), _p(eo),
                            _p(pr), _p(so)), "layout")
    R = int(ro[G])
    return dict(rank_mask=rm, rank_off=ro, disp_token=dtok[:R].copy(), expert_off=eo,
                perm_row=pr, slot_of=so, R=R)


def dispatch_rows(x, disp_token):
    """-> x_disp [R,d], same storage dtype as x (bit-exact copy)."""
    xx = np.ascontiguousarray(x)
    T, d = xx.shape
    dt = _c(disp_token, np.int32)
    out = np.empty((dt.shape[0], d), xx.dtype)
    _check(lib().orc_dispatch_rows(_p(xx), T, d, xx.itemsize, _p(dt), dt.shape[0], _p(out)),
           "dispatch")
    return out


def ffn_rows(x, src_row, expert, w_gate, w_up, w_down, want_h=False):
    """SwiGLU rows: y[i] = W_down[e] (silu(W_gate[e] a) * (W_up[e] a)), a = x[src_row[i]].

    -> y [n,d] float64 (and h [n,F] float64 if want_h).
    """
    xx = np.ascontiguousarray(x)
    dt = _dt(xx)
    wg, wu, wd = (np.ascontiguousarray(w) for w in (w_gate, w_up, w_down))
    for w in (wg, wu, wd):
        if w.dtype != xx.dtype:
            raise TypeError("weights and activations must share a dtype")
    E, F, d = wg.shape
    assert xx.shape[1] == d and wd.shape == (E, d, F) and wu.shape == wg.shape
    src = _c(src_row, np.int32)
    ex = _c(expert, np.int32)
    n = src.shape[0]
    if n and int(src.max()) >= xx.shape[0]:
        raise ValueError("src_row out of range")
    y = np.empty((n, d), np.float64)
    h = np.empty((n, F), np.float64) if want_h else None
    _check(lib().orc_ffn_rows(_p(xx), dt, d, F, n, _p(src), _p(ex), E, _p(wg), _p(wu), _p(wd),
                              _p(y), _p(h) if want_h else None), "ffn")
    return (y, h) if want_h else y


def combine(y, slot_of, gates, T, k):
    """-> out [T,d] float64."""
    yy = _c(y, np.float64)
    so = _c(slot_of, np.int32)
    g = _c(gates, np.float64)
    d = yy.shape[1]
    out = np.empty((T, d), np.float64)
    _check(lib().orc_combine(_p(yy), yy.shape[0], _p(so), _p(g), T, k, d, _p(out)), "combine")
    return out


# ---------------------------------------------------------------- whole layer

def slot_experts(expert_off):
    """Expert id of every slot, from the per-expert slot offsets."""
    eo = np.asarray(expert_off)
    return np.repeat(np.arange(eo.shape[0] - 1, dtype=np.int32), np.diff(eo)).astype(np.int32)


def layer(logits, x, place, G, k, w_gate, w_up, w_down, n_groups=1, topk_groups=1,
          want_h=False):
    """The whole hot path on one GPU's tokens, every intermediate returned."""
    E = np.asarray(logits).shape[1]
    T = np.asarray(logits).shape[0]
    idx, gates = route(logits, k, n_groups, topk_groups)
    C_ = coact(idx, E)
    lay = layout(idx, E, place, G)
    x_disp = dispatch_rows(x, lay["disp_token"])
    sexp = slot_experts(lay["expert_off"])
    # slot s reads dispatched row perm_row[s], a copy of token disp_token[perm_row[s]]
    r = ffn_rows(x_disp, lay["perm_row"], sexp, w_gate, w_up, w_down, want_h=want_h)
    y, h = (r if want_h else (r, None))
    out = combine(y, lay["slot_of"], gates, T, k)
    res = dict(topk_idx=idx, gates=gates, coact=C_, x_disp=x_disp, y=y, out=out, **lay)
    if want_h:
        res["h"] = h
    return res
