"""Host-side checks of the C ABI: the library loads, exports every declared
function, and rejects bad arguments before enqueuing any GPU work (none of
these calls touches a device, so they run without a GPU)."""
import ctypes as C

import pytest
import torch

from routing_dispatch_expert_top_amd import ops


@pytest.fixture(scope="module")
def L():
    return ops.lib()


def test_exports_every_declared_function(L):
    names = ops.header_functions()
    assert len(names) == 24
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.moe_abi_version() == 3
    assert ops.status_str(0) == "ok"
    assert "workspace" in ops.status_str(3)
    assert ops.status_str(99) == "unknown status"


def test_library_abi_must_match_the_header(L, monkeypatch):
    # the binding's signatures are the header's: a library of another ABI
    # version is refused when it is loaded
    assert ops.header_abi_version() == L.moe_abi_version()
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "header_abi_version", lambda: L.moe_abi_version() + 1)
    with pytest.raises(RuntimeError, match="rebuild"):
        ops.lib()


def test_workspace_bytes_host_only(L):
    a = ops.moe_dispatch_workspace_bytes(8192, 128, 8, 16)
    b = ops.moe_dispatch_workspace_bytes(16384, 128, 8, 16)
    assert 0 < a < b and a % 256 == 0
    assert ops.moe_dispatch_workspace_bytes(0, 8, 2, 4) > 0
    assert ops.moe_dispatch_workspace_bytes(-1, 8, 2, 4) == 0


NULL = None


@pytest.mark.parametrize("args,want", [
    ((NULL, 4, 8, 9, 1, 1, NULL, NULL, NULL), ops.MOE_ERR_ARG),          # k > E
    ((NULL, 4, 8, 0, 1, 1, NULL, NULL, NULL), ops.MOE_ERR_ARG),          # k < 1
    ((NULL, -1, 8, 2, 1, 1, NULL, NULL, NULL), ops.MOE_ERR_ARG),         # T < 0
    ((NULL, 4, 8, 2, 3, 1, NULL, NULL, NULL), ops.MOE_ERR_ARG),          # groups do not divide E
    ((NULL, 4, 8, 2, 4, 5, NULL, NULL, NULL), ops.MOE_ERR_ARG),          # topk_groups > n_groups
    ((NULL, 4, 8, 5, 4, 2, NULL, NULL, NULL), ops.MOE_ERR_ARG),          # < k eligible experts
    ((NULL, 4, 512, 2, 1, 1, NULL, NULL, NULL), ops.MOE_ERR_UNSUPPORTED),  # E > 256
    ((NULL, 4, 64, 17, 1, 1, NULL, NULL, NULL), ops.MOE_ERR_UNSUPPORTED),  # k > 16
    ((NULL, 4, 8, 2, 1, 1, NULL, NULL, NULL), ops.MOE_ERR_ARG),          # null pointers
    ((NULL, 0, 8, 2, 1, 1, NULL, NULL, NULL), ops.MOE_OK),               # empty: nothing to do
])
def test_route_argument_errors(L, args, want):
    assert L.moe_route(*args) == want


def test_validate_argument_errors(L):
    err = 16  # never dereferenced: every call below fails its argument check
    assert L.moe_validate_routing(NULL, NULL, -1, 8, 2, NULL, 4, err, NULL) == ops.MOE_ERR_ARG
    assert L.moe_validate_routing(NULL, NULL, 4, 8, 2, NULL, 4, NULL, NULL) == ops.MOE_ERR_ARG
    assert L.moe_validate_routing(NULL, NULL, 4, 0, 2, NULL, 4, err, NULL) == ops.MOE_ERR_ARG
    assert L.moe_validate_routing(NULL, NULL, 4, 64, 17, NULL, 4, err, NULL) == \
        ops.MOE_ERR_UNSUPPORTED


def test_coact_argument_errors(L):
    assert L.moe_coact_hist(NULL, 4, 8, 9, NULL, NULL) == ops.MOE_ERR_ARG
    assert L.moe_coact_hist(NULL, 4, 300, 2, NULL, NULL) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_coact_hist(NULL, 4, 8, 2, NULL, NULL) == ops.MOE_ERR_ARG
    assert L.moe_coact_hist(NULL, 0, 8, 2, NULL, NULL) == ops.MOE_OK
    assert L.moe_coact_hist(NULL, 4, 8, 1, NULL, NULL) == ops.MOE_OK   # k=1: no pairs


def _layout(L, T=4, E=8, k=2, G=4, place=1, ws=None, wsb=0, x=None, d=0, dt=1, ptr=1):
    p = ptr or None
    return L.moe_dispatch_layout(p, T, E, k, place or None, G, x, d, dt, p, p, p, p, p, p, p,
                                 ws, wsb, None)


def test_layout_argument_errors(L):
    assert _layout(L, G=0) == ops.MOE_ERR_ARG
    assert _layout(L, G=33) == ops.MOE_ERR_UNSUPPORTED
    assert _layout(L, k=9) == ops.MOE_ERR_ARG
    assert _layout(L, place=0) == ops.MOE_ERR_ARG
    assert _layout(L, ptr=0) == ops.MOE_ERR_ARG
    assert _layout(L) == ops.MOE_ERR_WORKSPACE                       # no workspace
    need = ops.moe_dispatch_workspace_bytes(4, 8, 2, 4)
    assert _layout(L, ws=16, wsb=need - 1) == ops.MOE_ERR_WORKSPACE  # too small
    assert _layout(L, ws=16, wsb=need, x=16, d=3) == ops.MOE_ERR_UNSUPPORTED  # row not 16B
    assert _layout(L, ws=16, wsb=need, x=16, d=64, dt=7) == ops.MOE_ERR_ARG   # bad dtype


def test_ffn_and_combine_argument_errors(L):
    p = 16
    W = L.moe_expert_workspace_bytes()
    assert W >= 64
    assert L.moe_expert_gate_up(p, p, p, 4, 8, 2, 100, 64, p, p, 1, p, p, W, None) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_gate_up(p, p, p, 4, 8, 2, 64, 96, p, p, 1, p, p, W, None) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_gate_up(None, p, p, 4, 8, 2, 64, 64, p, p, 1, p, p, W, None) == ops.MOE_ERR_ARG
    assert L.moe_expert_gate_up(p, p, p, 4, 8, 2, 64, 64, p, p, 5, p, p, W, None) == ops.MOE_ERR_ARG
    assert L.moe_expert_down(p, p, 4, 8, 9, 64, 64, p, 1, p, p, W, None) == ops.MOE_ERR_ARG
    assert L.moe_expert_down(None, p, 4, 8, 2, 64, 64, p, 1, p, p, W, None) == ops.MOE_ERR_ARG
    assert L.moe_grouped_ffn(p, p, p, 0, 8, 2, 64, 64, p, p, p, 1, p, p, p, W, None) == ops.MOE_OK
    # the workspace (the persistent launches' tile queue) is checked before any launch
    assert L.moe_expert_gate_up(p, p, p, 4, 8, 2, 64, 64, p, p, 1, p, None, W, None) == ops.MOE_ERR_WORKSPACE
    assert L.moe_expert_gate_up(p, p, p, 4, 8, 2, 64, 64, p, p, 1, p, p, W - 1, None) == ops.MOE_ERR_WORKSPACE
    assert L.moe_expert_down(p, p, 4, 8, 2, 64, 64, p, 1, p, None, W, None) == ops.MOE_ERR_WORKSPACE
    assert L.moe_expert_down(p, p, 4, 8, 2, 64, 64, p, 1, p, 8, W, None) == ops.MOE_ERR_WORKSPACE  # unaligned
    # bf16 operands addressed with 32-bit offsets: 2^20 * 8 slots x 4096 bf16
    # activations (64 GiB) and a 2^20 x 4096 weight panel are refused up front
    big_t = 1 << 20
    assert L.moe_expert_gate_up(p, p, p, big_t, 8, 8, 4096, 64, p, p, 1, p, p, W, None) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_down(p, p, big_t, 8, 8, 64, 4096, p, 1, p, p, W, None) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_gate_up(p, p, p, 4, 8, 2, 4096, 1 << 20, p, p, 1, p, p, W, None) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(p, p, p, 4, 0, 64, 1, p, None) == ops.MOE_ERR_ARG
    assert L.moe_combine(p, p, p, 4, 2, 4, 1, p, None) == ops.MOE_ERR_UNSUPPORTED  # 8-byte rows
    assert L.moe_combine(None, p, p, 4, 2, 64, 1, p, None) == ops.MOE_ERR_ARG
    assert L.moe_combine(p, p, p, 0, 2, 64, 1, p, None) == ops.MOE_OK


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        ops.moe_route(torch.zeros(4, 8), 2)


def test_backward_expert_calls_need_their_workspace():
    """bf16 expert backward calls check their workspace before any launch
    (pointers are never dereferenced on this path)."""
    L = ops.lib()
    fake = 0x10000  # 16-byte aligned, never read: the call returns first
    T, E, k, d, F = 16, 4, 2, 64, 64
    need = L.moe_expert_bwd_workspace_bytes(T, E, k, d, F)
    assert need > 0
    st = L.moe_expert_down_bwd(fake, fake, fake, fake, T, E, k, d, F, fake, ops.MOE_BF16, fake,
                               fake, None, 0, None)
    assert st == ops.MOE_ERR_WORKSPACE
    st = L.moe_expert_gate_up_bwd(fake, fake, fake, fake, T, E, k, d, F, fake, fake, ops.MOE_BF16,
                                  fake, fake, fake, fake, need - 1, None)
    assert st == ops.MOE_ERR_WORKSPACE
    st = L.moe_expert_down_bwd(fake, fake, fake, fake, T, E, k, 96, F, fake, ops.MOE_BF16, fake,
                               fake, fake, need, None)
    assert st == ops.MOE_ERR_UNSUPPORTED  # d not a multiple of 64


def test_binding_refuses_undersized_or_mistyped_buffers(L):
    # The C ABI takes raw pointers; the binding checks every buffer's size and
    # element type before the call (host tensors here: the checks come first).
    T, k, E, d, F = 8, 2, 4, 64, 64
    i32, f32, bf = torch.int32, torch.float32, torch.bfloat16
    slot_of = torch.zeros(T * k, dtype=i32)
    gates = torch.zeros(T * k, dtype=f32)
    y = torch.zeros(T * k, d, dtype=bf)
    with pytest.raises(ValueError, match="out holds"):
        ops.moe_combine(y, slot_of, gates, T, k, out=torch.zeros(T - 1, d, dtype=bf))
    with pytest.raises(TypeError, match="slot_of must be"):
        ops.moe_combine(y, slot_of.long(), gates, T, k, out=torch.zeros(T, d, dtype=bf))
    logits = torch.zeros(T, E, dtype=f32)
    with pytest.raises(ValueError, match="gates holds"):
        ops.moe_route(logits, k, gates=torch.zeros(T * k - 1, dtype=f32))
    x_disp = torch.zeros(T * k, d, dtype=bf)
    wg = torch.zeros(E, F, d, dtype=bf)
    with pytest.raises(ValueError, match="w_up must be"):
        ops.moe_expert_gate_up(x_disp, slot_of, torch.zeros(E + 1, dtype=i32), T, k, wg,
                               torch.zeros(E, F + 64, d, dtype=bf), workspace=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(TypeError, match="w_gate must be"):
        ops.moe_expert_gate_up(x_disp, slot_of, torch.zeros(E + 1, dtype=i32), T, k, wg.float(),
                               wg.float(), workspace=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="expert_off holds"):
        ops.moe_expert_down(torch.zeros(T * k, F, dtype=bf), torch.zeros(E, dtype=i32), T, k,
                            torch.zeros(E, d, F, dtype=bf), workspace=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="whole rows"):  # slot rows: width and type only
        ops.moe_expert_down(torch.zeros(T * k, F, dtype=bf), torch.zeros(E + 1, dtype=i32), T, k,
                            torch.zeros(E, d, F, dtype=bf), y=torch.zeros(T * k * d + 3, dtype=bf),
                            workspace=torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="dw_down holds"):
        ops.moe_expert_down_bwd(y, torch.zeros(T * k, F, dtype=bf), torch.zeros(T * k, 2 * F, dtype=bf),
                                torch.zeros(E + 1, dtype=i32), T, k, torch.zeros(E, d, F, dtype=bf),
                                dw_down=torch.zeros(E * d * F - 1, dtype=f32),
                                workspace=torch.zeros(1, dtype=torch.uint8))
    topk = torch.zeros(T, k, dtype=i32)
    out = ops.alloc_layout(T, E, k, 2, "cpu", d, bf)
    out["perm_row"] = out["perm_row"][:-1]
    with pytest.raises(ValueError, match="perm_row holds"):
        ops.moe_dispatch_layout(topk, E, torch.zeros(E, dtype=i32), 2,
                                x=torch.zeros(T, d, dtype=bf), out=out)
