"""Python binding of libmoe (include/moe.h): argument marshalling only.

Each function has the name of the C entry point it calls, takes torch device
tensors (torch is used for device memory and streams only), allocates any
output that is not passed in, and raises ``MoeError`` on a non-OK status.
Every step of the hot path runs in the HIP kernels of libmoe.so; there is no
fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "moe.h")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_F32, MOE_BF16 = 0, 1

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} (status {status})")


def lib():
    """Load libmoe.so (built in-tree); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        p, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        sig = {
            "moe_abi_version": (C.c_int, []),
            "moe_status_str": (C.c_char_p, [C.c_int]),
            "moe_route": (C.c_int, [p, i32, i32, i32, i32, i32, p, p, p]),
            "moe_coact_hist": (C.c_int, [p, i32, i32, i32, p, p]),
            "moe_dispatch_workspace_bytes": (sz, [i32, i32, i32, i32]),
            "moe_dispatch_layout": (C.c_int, [p, i32, i32, i32, p, i32, p, i32, C.c_int,
                                              p, p, p, p, p, p, p, p, sz, p]),
            "moe_expert_workspace_bytes": (sz, []),
            "moe_expert_gate_up": (C.c_int, [p, p, p, i32, i32, i32, i32, i32, p, p, C.c_int,
                                             p, p, sz, p]),
            "moe_expert_down": (C.c_int, [p, p, i32, i32, i32, i32, i32, p, C.c_int, p, p, sz,
                                          p]),
            "moe_grouped_ffn": (C.c_int, [p, p, p, i32, i32, i32, i32, i32, p, p, p, C.c_int,
                                          p, p, p, sz, p]),
            "moe_combine": (C.c_int, [p, p, p, i32, i32, i32, C.c_int, p, p]),
            "moe_plan_placement": (C.c_int, [p, p, i32, i32, i32, i32, p]),
            "moe_expert_gate_up_save": (C.c_int, [p, p, p, i32, i32, i32, i32, i32, p, p,
                                                  C.c_int, p, p, p, sz, p]),
            "moe_combine_bwd": (C.c_int, [p, p, p, p, i32, i32, i32, C.c_int, p, p, p]),
            "moe_expert_bwd_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
            "moe_expert_down_bwd": (C.c_int, [p, p, p, p, i32, i32, i32, i32, i32, p, C.c_int,
                                              p, p, p, sz, p]),
            "moe_expert_gate_up_bwd": (C.c_int, [p, p, p, p, i32, i32, i32, i32, i32, p, p,
                                                 C.c_int, p, p, p, p, sz, p]),
            "moe_dispatch_bwd": (C.c_int, [p, p, i32, i32, i32, C.c_int, p, p]),
            "moe_route_bwd": (C.c_int, [p, p, p, i32, i32, i32, p, p]),
            "moe_shuffle_workspace_bytes": (sz, [i32, i32]),
            "moe_token_shuffle": (C.c_int, [p, i32, i32, i32, p, i32, p, i32, C.c_int, p, p, p,
                                            p, p, p, sz, p]),
            "moe_replica_layout": (C.c_int, [p, i32, i32, i32, p, i32, i32, p, i32, C.c_int,
                                             p, p, p, p, p, p, p, p, p, p, sz, p]),
            "moe_validate_routing": (C.c_int, [p, p, i32, i32, i32, p, i32, p, p]),
            "moe_dispatch_layout_noalloc": (C.c_int, [p, i32, i32, i32, p, i32, p, i32,
                                                      C.c_int, p, p, p, p, p, p, p, p]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        # The signatures above are those of include/moe.h: a library built
        # from another version of it would be called with the wrong arguments.
        want, got = header_abi_version(), L.moe_abi_version()
        if got != want:
            raise RuntimeError(f"{LIB_PATH} implements ABI {got} but include/moe.h declares "
                               f"ABI {want}: rebuild it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        _lib = L
    return _lib


def header_abi_version() -> int:
    """MOE_ABI_VERSION as include/moe.h defines it."""
    m = re.search(r"#define\s+MOE_ABI_VERSION\s+(\d+)", open(HEADER).read())
    if m is None:
        raise RuntimeError(f"{HEADER} defines no MOE_ABI_VERSION")
    return int(m.group(1))


def header_functions():
    """Names of the functions include/moe.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", txt)))


def status_str(s: int) -> str:
    return lib().moe_status_str(int(s)).decode()


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


_I32, _F32 = torch.int32, torch.float32


def _need(fn, name, t, numel, dtype=None):
    """Refuse a tensor the call would read or write past its end (the C ABI
    takes raw pointers and cannot check), or one of the wrong element type."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{fn}: {name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{fn}: {name} must be {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{fn}: {name} holds {t.numel()} elements, the call uses {numel}")


def _rows(fn, name, t, width, dtype=None):
    """A buffer of slot rows: how many the call touches (expert_off[E], at
    most T*k) is known only on the device, so only the row width and the
    element type are checked."""
    if t is None:
        return
    _need(fn, name, t, 0, dtype)
    if t.numel() % width:
        raise ValueError(f"{fn}: {name} must hold whole rows of {width} elements")


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"activations and weights must be float32 or bfloat16, got {t.dtype}")


# ---------------------------------------------------------------- entry points

def moe_route(logits, k, n_groups=1, topk_groups=1, topk_idx=None, gates=None, stream=None):
    T, E = logits.shape
    dev = logits.device
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    gates = torch.empty((T, k), dtype=torch.float32, device=dev) if gates is None else gates
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    _need("moe_route", "topk_idx", topk_idx, T * k, _I32)
    _need("moe_route", "gates", gates, T * k, _F32)
    _check("moe_route", lib().moe_route(_ptr(logits), T, E, k, n_groups, topk_groups,
                                        _ptr(topk_idx), _ptr(gates), _stream(stream)))
    return topk_idx, gates


def moe_coact_hist(topk_idx, E, coact=None, stream=None):
    T, k = topk_idx.shape
    coact = torch.zeros((E, E), dtype=torch.int32, device=topk_idx.device) if coact is None else coact
    _need("moe_coact_hist", "topk_idx", topk_idx, T * k, _I32)
    _need("moe_coact_hist", "coact", coact, E * E, _I32)
    _check("moe_coact_hist", lib().moe_coact_hist(_ptr(topk_idx), T, E, k, _ptr(coact),
                                                  _stream(stream)))
    return coact


def moe_dispatch_workspace_bytes(T, E, k, G):
    return int(lib().moe_dispatch_workspace_bytes(T, E, k, G))


def alloc_layout(T, E, k, G, device, d=None, dtype=None):
    """Output buffers of moe_dispatch_layout, sized for the T*k upper bound,
    and its workspace (zero-filled before its first use, as the call needs;
    every call leaves it so)."""
    i32 = dict(dtype=torch.int32, device=device)
    out = dict(rank_mask=torch.empty(T, dtype=torch.int32, device=device),
               rank_off=torch.empty(G + 1, **i32), disp_token=torch.empty(T * k, **i32),
               expert_off=torch.empty(E + 1, **i32), perm_row=torch.empty(T * k, **i32),
               slot_of=torch.empty(T * k, **i32),
               workspace=torch.zeros(max(1, moe_dispatch_workspace_bytes(T, E, k, G)),
                                     dtype=torch.uint8, device=device))
    if d is not None:
        out["x_disp"] = torch.empty((T * k, d), dtype=dtype, device=device)
    return out


def _need_layout(fn, topk_idx, E, place, G, x, out):
    T, k = topk_idx.shape
    _need(fn, "topk_idx", topk_idx, T * k, _I32)
    _need(fn, "place", place, E, _I32)
    for name, n in (("rank_mask", T), ("rank_off", G + 1), ("disp_token", T * k),
                    ("expert_off", E + 1), ("perm_row", T * k), ("slot_of", T * k)):
        _need(fn, name, out[name], n, _I32)
    if x is not None:
        if x.dim() != 2 or x.shape[0] != T:
            raise ValueError(f"{fn}: x must be [T, d] with T = {T}")
        _need(fn, "x_disp", out.get("x_disp"), T * k * x.shape[1], x.dtype)
        if out.get("x_disp") is None:
            raise ValueError(f"{fn}: x given without an x_disp buffer")


def moe_dispatch_layout(topk_idx, E, place, G, x=None, out=None, stream=None):
    """Returns the dict of outputs (rank_mask holds uint32 bits in an int32 tensor)."""
    T, k = topk_idx.shape
    d = x.shape[1] if x is not None else None
    if out is None:
        out = alloc_layout(T, E, k, G, topk_idx.device, d, x.dtype if x is not None else None)
    dt = dtype_code(x) if x is not None else MOE_F32
    _need_layout("moe_dispatch_layout", topk_idx, E, place, G, x, out)
    ws = out["workspace"]
    _check("moe_dispatch_layout", lib().moe_dispatch_layout(
        _ptr(topk_idx), T, E, k, _ptr(place), G, _ptr(x), d or 0, dt,
        _ptr(out["rank_mask"]), _ptr(out["rank_off"]), _ptr(out["disp_token"]),
        _ptr(out["expert_off"]), _ptr(out["perm_row"]), _ptr(out["slot_of"]),
        _ptr(out.get("x_disp")) if x is not None else None, _ptr(ws), ws.numel(),
        _stream(stream)))
    return out


def moe_dispatch_layout_noalloc(topk_idx, E, place, G, x=None, out=None, stream=None):
    """moe_dispatch_layout on the library's own scratch (no workspace); with
    `out` given (a dict of alloc_layout's buffers) nothing is allocated."""
    T, k = topk_idx.shape
    d = x.shape[1] if x is not None else None
    if out is None:
        out = alloc_layout(T, E, k, G, topk_idx.device, d, x.dtype if x is not None else None)
    dt = dtype_code(x) if x is not None else MOE_F32
    _need_layout("moe_dispatch_layout_noalloc", topk_idx, E, place, G, x, out)
    _check("moe_dispatch_layout_noalloc", lib().moe_dispatch_layout_noalloc(
        _ptr(topk_idx), T, E, k, _ptr(place), G, _ptr(x), d or 0, dt,
        _ptr(out["rank_mask"]), _ptr(out["rank_off"]), _ptr(out["disp_token"]),
        _ptr(out["expert_off"]), _ptr(out["perm_row"]), _ptr(out["slot_of"]),
        _ptr(out.get("x_disp")) if x is not None else None, _stream(stream)))
    return out


def moe_replica_layout(topk_idx, E, rep_mask, G, ranks_per_node, x=None, out=None,
                       stream=None):
    """rep_mask [E] int32 device tensor (uint32 bits: ranks holding a copy of
    expert e). Returns the layout dict of moe_dispatch_layout plus rank_of
    [T*k] and node_mask [T] (uint32 bits in an int32 tensor)."""
    T, k = topk_idx.shape
    d = x.shape[1] if x is not None else None
    dev = topk_idx.device
    if out is None:
        out = alloc_layout(T, E, k, G, dev, d, x.dtype if x is not None else None)
    if "rank_of" not in out:
        out["rank_of"] = torch.empty(T * k, dtype=torch.int32, device=dev)
        out["node_mask"] = torch.empty(T, dtype=torch.int32, device=dev)
    dt = dtype_code(x) if x is not None else MOE_F32
    _need_layout("moe_replica_layout", topk_idx, E, None, G, x, out)
    _need("moe_replica_layout", "rep_mask", rep_mask, E, _I32)
    _need("moe_replica_layout", "rank_of", out["rank_of"], T * k, _I32)
    _need("moe_replica_layout", "node_mask", out["node_mask"], T, _I32)
    ws = out["workspace"]
    _check("moe_replica_layout", lib().moe_replica_layout(
        _ptr(topk_idx), T, E, k, _ptr(rep_mask), G, ranks_per_node, _ptr(x), d or 0, dt,
        _ptr(out["rank_of"]), _ptr(out["node_mask"]),
        _ptr(out["rank_mask"]), _ptr(out["rank_off"]), _ptr(out["disp_token"]),
        _ptr(out["expert_off"]), _ptr(out["perm_row"]), _ptr(out["slot_of"]),
        _ptr(out.get("x_disp")) if x is not None else None, _ptr(ws), ws.numel(),
        _stream(stream)))
    return out


def moe_token_shuffle(want_idx, aff, x=None, out=None, stream=None):
    """want_idx [T,k] int32, aff [E,G] int32 device tensors. Returns a dict
    with dest, rank_off, perm, pos (and x_shuf if x is given)."""
    T, k = want_idx.shape
    E, G = aff.shape
    dev = want_idx.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(dest=torch.empty(T, **i32), rank_off=torch.empty(G + 1, **i32),
                   perm=torch.empty(T, **i32), pos=torch.empty(T, **i32),
                   workspace=torch.zeros(max(1, int(lib().moe_shuffle_workspace_bytes(T, G))),
                                         dtype=torch.uint8, device=dev))
        if x is not None:
            out["x_shuf"] = torch.empty_like(x)
    dt = dtype_code(x) if x is not None else MOE_F32
    fn = "moe_token_shuffle"
    _need(fn, "want_idx", want_idx, T * k, _I32)
    _need(fn, "aff", aff, E * G, _I32)
    for name in ("dest", "perm", "pos"):
        _need(fn, name, out[name], T, _I32)
    _need(fn, "rank_off", out["rank_off"], G + 1, _I32)
    if x is not None:
        if x.dim() != 2 or x.shape[0] != T:
            raise ValueError(f"{fn}: x must be [T, d] with T = {T}")
        if out.get("x_shuf") is None:
            raise ValueError(f"{fn}: x given without an x_shuf buffer")
        _need(fn, "x_shuf", out["x_shuf"], x.numel(), x.dtype)
    ws = out["workspace"]
    _check("moe_token_shuffle", lib().moe_token_shuffle(
        _ptr(want_idx), T, E, k, _ptr(aff), G, _ptr(x), x.shape[1] if x is not None else 0, dt,
        _ptr(out["dest"]), _ptr(out["rank_off"]), _ptr(out["perm"]), _ptr(out["pos"]),
        _ptr(out.get("x_shuf")) if x is not None else None, _ptr(ws), ws.numel(),
        _stream(stream)))
    return out


def expert_workspace(device):
    """A zero-filled workspace for the forward expert calls (they leave it
    zero-filled, so one buffer serves every call on one stream)."""
    return torch.zeros(max(16, int(lib().moe_expert_workspace_bytes())), dtype=torch.uint8,
                       device=device)


def _need_gate_up(fn, x_disp, perm_row, expert_off, T, k, w_gate, w_up):
    E, F, d = w_gate.shape
    dt = x_disp.dtype
    if tuple(w_up.shape) != (E, F, d):
        raise ValueError(f"{fn}: w_up must be [E, F, d] like w_gate")
    if x_disp.dim() != 2 or x_disp.shape[1] != d:
        raise ValueError(f"{fn}: x_disp must be [rows, d] with d = {d}")
    _need(fn, "w_gate", w_gate, 0, dt)
    _need(fn, "w_up", w_up, 0, dt)
    _need(fn, "perm_row", perm_row, T * k, _I32)
    _need(fn, "expert_off", expert_off, E + 1, _I32)


def _need_down(fn, h, expert_off, T, k, w_down):
    E, d, F = w_down.shape
    _rows(fn, "h", h, F)
    _need(fn, "w_down", w_down, 0, h.dtype)
    _need(fn, "expert_off", expert_off, E + 1, _I32)


def moe_expert_gate_up(x_disp, perm_row, expert_off, T, k, w_gate, w_up, h=None, workspace=None,
                       stream=None):
    E, F, d = w_gate.shape
    h = torch.empty((T * k, F), dtype=x_disp.dtype, device=x_disp.device) if h is None else h
    ws = expert_workspace(x_disp.device) if workspace is None else workspace
    _need_gate_up("moe_expert_gate_up", x_disp, perm_row, expert_off, T, k, w_gate, w_up)
    _rows("moe_expert_gate_up", "h", h, F, x_disp.dtype)
    _check("moe_expert_gate_up", lib().moe_expert_gate_up(
        _ptr(x_disp), _ptr(perm_row), _ptr(expert_off), T, E, k, d, F, _ptr(w_gate), _ptr(w_up),
        dtype_code(x_disp), _ptr(h), _ptr(ws), ws.numel(), _stream(stream)))
    return h


def moe_expert_down(h, expert_off, T, k, w_down, y=None, workspace=None, stream=None):
    E, d, F = w_down.shape
    y = torch.empty((T * k, d), dtype=h.dtype, device=h.device) if y is None else y
    ws = expert_workspace(h.device) if workspace is None else workspace
    _need_down("moe_expert_down", h, expert_off, T, k, w_down)
    _rows("moe_expert_down", "y", y, d, h.dtype)
    _check("moe_expert_down", lib().moe_expert_down(
        _ptr(h), _ptr(expert_off), T, E, k, d, F, _ptr(w_down), dtype_code(h), _ptr(y), _ptr(ws),
        ws.numel(), _stream(stream)))
    return y


def moe_grouped_ffn(x_disp, perm_row, expert_off, T, k, w_gate, w_up, w_down, h=None, y=None,
                    workspace=None, stream=None):
    E, F, d = w_gate.shape
    dev, dt = x_disp.device, x_disp.dtype
    h = torch.empty((T * k, F), dtype=dt, device=dev) if h is None else h
    y = torch.empty((T * k, d), dtype=dt, device=dev) if y is None else y
    ws = expert_workspace(dev) if workspace is None else workspace
    _need_gate_up("moe_grouped_ffn", x_disp, perm_row, expert_off, T, k, w_gate, w_up)
    if tuple(w_down.shape) != (E, d, F):
        raise ValueError("moe_grouped_ffn: w_down must be [E, d, F]")
    _need("moe_grouped_ffn", "w_down", w_down, 0, dt)
    _rows("moe_grouped_ffn", "h", h, F, dt)
    _rows("moe_grouped_ffn", "y", y, d, dt)
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _ptr(x_disp), _ptr(perm_row), _ptr(expert_off), T, E, k, d, F, _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), dtype_code(x_disp), _ptr(h), _ptr(y), _ptr(ws), ws.numel(),
        _stream(stream)))
    return h, y


# ---------------------------------------------------------------- backward

def moe_expert_gate_up_save(x_disp, perm_row, expert_off, T, k, w_gate, w_up, h=None, uv=None,
                            workspace=None, stream=None):
    E, F, d = w_gate.shape
    dev, dt = x_disp.device, x_disp.dtype
    h = torch.empty((T * k, F), dtype=dt, device=dev) if h is None else h
    uv = torch.empty((T * k, 2 * F), dtype=dt, device=dev) if uv is None else uv
    ws = expert_workspace(dev) if workspace is None else workspace
    _need_gate_up("moe_expert_gate_up_save", x_disp, perm_row, expert_off, T, k, w_gate, w_up)
    _rows("moe_expert_gate_up_save", "h", h, F, dt)
    _rows("moe_expert_gate_up_save", "uv", uv, 2 * F, dt)
    _check("moe_expert_gate_up_save", lib().moe_expert_gate_up_save(
        _ptr(x_disp), _ptr(perm_row), _ptr(expert_off), T, E, k, d, F, _ptr(w_gate), _ptr(w_up),
        dtype_code(x_disp), _ptr(h), _ptr(uv), _ptr(ws), ws.numel(), _stream(stream)))
    return h, uv


def moe_combine_bwd(dout, y, slot_of, gates, T, k, dy=None, dgates=None, stream=None):
    d = dout.shape[1]
    dy = torch.empty((T * k, d), dtype=dout.dtype, device=dout.device) if dy is None else dy
    dgates = (torch.empty((T, k), dtype=torch.float32, device=dout.device)
              if dgates is None else dgates)
    fn = "moe_combine_bwd"
    if dout.dim() != 2 or dout.shape[0] != T:
        raise ValueError(f"{fn}: dout must be [T, d] with T = {T}")
    _rows(fn, "y", y, d, dout.dtype)
    _need(fn, "slot_of", slot_of, T * k, _I32)
    _need(fn, "gates", gates, T * k, _F32)
    _rows(fn, "dy", dy, d, dout.dtype)
    _need(fn, "dgates", dgates, T * k, _F32)
    _check("moe_combine_bwd", lib().moe_combine_bwd(
        _ptr(dout), _ptr(y), _ptr(slot_of), _ptr(gates), T, k, d, dtype_code(dout), _ptr(dy),
        _ptr(dgates), _stream(stream)))
    return dy, dgates


def moe_expert_bwd_workspace_bytes(T, E, k, d, F):
    return int(lib().moe_expert_bwd_workspace_bytes(T, E, k, d, F))


def bwd_workspace(T, E, k, d, F, device):
    return torch.empty(max(1, moe_expert_bwd_workspace_bytes(T, E, k, d, F)), dtype=torch.uint8,
                       device=device)


def moe_expert_down_bwd(dy, h, uv, expert_off, T, k, w_down, duv=None, dw_down=None,
                        workspace=None, stream=None):
    E, d, F = w_down.shape
    dev = dy.device
    duv = torch.empty((T * k, 2 * F), dtype=dy.dtype, device=dev) if duv is None else duv
    dw_down = (torch.empty((E, d, F), dtype=torch.float32, device=dev)
               if dw_down is None else dw_down)
    ws = bwd_workspace(T, E, k, d, F, dev) if workspace is None else workspace
    fn = "moe_expert_down_bwd"
    _need_down(fn, h, expert_off, T, k, w_down)
    _rows(fn, "dy", dy, d, h.dtype)
    _rows(fn, "uv", uv, 2 * F, h.dtype)
    _rows(fn, "duv", duv, 2 * F, h.dtype)
    _need(fn, "dw_down", dw_down, E * d * F, _F32)
    _check("moe_expert_down_bwd", lib().moe_expert_down_bwd(
        _ptr(dy), _ptr(h), _ptr(uv), _ptr(expert_off), T, E, k, d, F, _ptr(w_down),
        dtype_code(dy), _ptr(duv), _ptr(dw_down), _ptr(ws), ws.numel(), _stream(stream)))
    return duv, dw_down


def moe_expert_gate_up_bwd(duv, x_disp, perm_row, expert_off, T, k, w_gate, w_up, da=None,
                           dw_gate=None, dw_up=None, workspace=None, stream=None):
    E, F, d = w_gate.shape
    dev = duv.device
    da = torch.empty((T * k, d), dtype=duv.dtype, device=dev) if da is None else da
    f32 = dict(dtype=torch.float32, device=dev)
    dw_gate = torch.empty((E, F, d), **f32) if dw_gate is None else dw_gate
    dw_up = torch.empty((E, F, d), **f32) if dw_up is None else dw_up
    ws = bwd_workspace(T, E, k, d, F, dev) if workspace is None else workspace
    fn = "moe_expert_gate_up_bwd"
    _need_gate_up(fn, x_disp, perm_row, expert_off, T, k, w_gate, w_up)
    _rows(fn, "duv", duv, 2 * F, x_disp.dtype)
    _rows(fn, "da", da, d, x_disp.dtype)
    _need(fn, "dw_gate", dw_gate, E * F * d, _F32)
    _need(fn, "dw_up", dw_up, E * F * d, _F32)
    _check("moe_expert_gate_up_bwd", lib().moe_expert_gate_up_bwd(
        _ptr(duv), _ptr(x_disp), _ptr(perm_row), _ptr(expert_off), T, E, k, d, F, _ptr(w_gate),
        _ptr(w_up), dtype_code(duv), _ptr(da), _ptr(dw_gate), _ptr(dw_up), _ptr(ws), ws.numel(),
        _stream(stream)))
    return da, dw_gate, dw_up


def moe_dispatch_bwd(da, slot_of, T, k, dx=None, stream=None):
    d = da.shape[1]
    dx = torch.empty((T, d), dtype=da.dtype, device=da.device) if dx is None else dx
    _rows("moe_dispatch_bwd", "da", da, d)
    _need("moe_dispatch_bwd", "slot_of", slot_of, T * k, _I32)
    _need("moe_dispatch_bwd", "dx", dx, T * d, da.dtype)
    _check("moe_dispatch_bwd", lib().moe_dispatch_bwd(
        _ptr(da), _ptr(slot_of), T, k, d, dtype_code(da), _ptr(dx), _stream(stream)))
    return dx


def moe_route_bwd(gates, dgates, topk_idx, E, dlogits=None, stream=None):
    T, k = gates.shape
    dlogits = (torch.empty((T, E), dtype=torch.float32, device=gates.device)
               if dlogits is None else dlogits)
    _need("moe_route_bwd", "gates", gates, T * k, _F32)
    _need("moe_route_bwd", "dgates", dgates, T * k, _F32)
    _need("moe_route_bwd", "topk_idx", topk_idx, T * k, _I32)
    _need("moe_route_bwd", "dlogits", dlogits, T * E, _F32)
    _check("moe_route_bwd", lib().moe_route_bwd(
        _ptr(gates), _ptr(dgates), _ptr(topk_idx), T, E, k, _ptr(dlogits), _stream(stream)))
    return dlogits


MOE_BAD_LOGIT, MOE_BAD_EXPERT, MOE_BAD_REPEAT, MOE_BAD_RANK = 1, 2, 4, 8
_BAD_NAMES = {MOE_BAD_LOGIT: "NaN logit", MOE_BAD_EXPERT: "expert id outside [0,E)",
              MOE_BAD_REPEAT: "expert repeated within a token",
              MOE_BAD_RANK: "rank outside [0,G)"}


def moe_validate_routing(logits, topk_idx, E, place=None, G=1, stream=None):
    """Device-side check of routing inputs; synchronises the stream and
    returns the flags found (0: nothing wrong). logits / topk_idx / place may
    each be None to skip that check."""
    T, k = topk_idx.shape if topk_idx is not None else (logits.shape[0], 1)
    ref = next(a for a in (logits, topk_idx, place) if a is not None)
    err = torch.zeros(1, dtype=torch.int32, device=ref.device)
    _need("moe_validate_routing", "logits", logits, T * E, _F32)
    _need("moe_validate_routing", "topk_idx", topk_idx, T * k, _I32)
    _need("moe_validate_routing", "place", place, E, _I32)
    _check("moe_validate_routing", lib().moe_validate_routing(
        _ptr(logits), _ptr(topk_idx), T, E, k, _ptr(place), G, _ptr(err), _stream(stream)))
    torch.cuda.synchronize(ref.device)  # the kernel may run on another stream than torch's
    return int(err.cpu().item()) & 0xFFFFFFFF


def bad_routing_names(flags: int):
    return [n for b, n in _BAD_NAMES.items() if flags & b]


def debug_enabled() -> bool:
    return os.environ.get("MOE_DEBUG", "0") not in ("", "0")


def moe_plan_placement(coact, load, G, ranks_per_node=1, swap_passes=8):
    """Host call: coact [E,E] and load [E] (array-likes, converted to int64
    host arrays; device tensors are copied to the host first) -> place [E]
    int32 numpy array."""
    import numpy as np

    def host64(a):
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
        return np.ascontiguousarray(np.asarray(a, dtype=np.int64))

    c, ld = host64(coact), host64(load)
    E = ld.shape[0]
    if c.shape != (E, E):
        raise ValueError("coact must be [E,E] with E = len(load)")
    place = np.empty(E, dtype=np.int32)
    _check("moe_plan_placement", lib().moe_plan_placement(
        c.ctypes.data, ld.ctypes.data, E, G, ranks_per_node, swap_passes, place.ctypes.data))
    return place


def moe_combine(y, slot_of, gates, T, k, out=None, stream=None):
    d = y.shape[1]
    out = torch.empty((T, d), dtype=y.dtype, device=y.device) if out is None else out
    _rows("moe_combine", "y", y, d)
    _need("moe_combine", "slot_of", slot_of, T * k, _I32)
    _need("moe_combine", "gates", gates, T * k, _F32)
    _need("moe_combine", "out", out, T * d, y.dtype)
    _check("moe_combine", lib().moe_combine(_ptr(y), _ptr(slot_of), _ptr(gates), T, k, d,
                                            dtype_code(y), _ptr(out), _stream(stream)))
    return out


# ---------------------------------------------------------------- whole layer

class Layer:
    """Preallocated buffers for repeated passes of the hot path on one shape."""

    def __init__(self, T, d, E, k, F, G, dtype, device, n_groups=1, topk_groups=1):
        self.T, self.d, self.E, self.k, self.F, self.G = T, d, E, k, F, G
        self.n_groups, self.topk_groups = n_groups, topk_groups
        dev = torch.device(device)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.gates = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.coact = torch.zeros((E, E), dtype=torch.int32, device=dev)
        self.lay = alloc_layout(T, E, k, G, dev, d, dtype)
        self.h = torch.empty((T * k, F), dtype=dtype, device=dev)
        self.expert_ws = expert_workspace(dev)
        self.y = torch.empty((T * k, d), dtype=dtype, device=dev)
        self.out = torch.empty((T, d), dtype=dtype, device=dev)

    def route(self, logits, stream=None):
        moe_route(logits, self.k, self.n_groups, self.topk_groups, self.topk_idx, self.gates,
                  stream)

    def coact_hist(self, stream=None):
        moe_coact_hist(self.topk_idx, self.E, self.coact, stream)

    def dispatch(self, x, place, stream=None):
        moe_dispatch_layout(self.topk_idx, self.E, place, self.G, x, self.lay, stream)

    def gate_up(self, w_gate, w_up, stream=None):
        moe_expert_gate_up(self.lay["x_disp"], self.lay["perm_row"], self.lay["expert_off"],
                           self.T, self.k, w_gate, w_up, self.h, self.expert_ws, stream)

    def down(self, w_down, stream=None):
        moe_expert_down(self.h, self.lay["expert_off"], self.T, self.k, w_down, self.y,
                        self.expert_ws, stream)

    def combine(self, stream=None):
        moe_combine(self.y, self.lay["slot_of"], self.gates, self.T, self.k, self.out, stream)

    def validate(self, logits, place, stream=None):
        """MOE_DEBUG: check logits, the routing result and the placement on
        the device; raise ValueError naming what is wrong."""
        flags = moe_validate_routing(logits, self.topk_idx, self.E, place, self.G, stream)
        if flags:
            raise ValueError("invalid routing inputs: " + ", ".join(bad_routing_names(flags)))

    def forward(self, logits, x, place, w_gate, w_up, w_down, stream=None):
        """One pass of the whole hot path; the co-activation counts accumulate.
        With MOE_DEBUG=1 in the environment the routing inputs are validated
        on the device after routing (this synchronises)."""
        self.route(logits, stream)
        if debug_enabled():
            self.validate(logits, place, stream)
        self.coact_hist(stream)
        self.dispatch(x, place, stream)
        self.gate_up(w_gate, w_up, stream)
        self.down(w_down, stream)
        self.combine(stream)
        return self.out
