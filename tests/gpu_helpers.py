"""Helpers of the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, download every output, compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

from routing_dispatch_expert_top_amd import ops, synth

# Tolerances: max|gpu - ref| <= tau * max|ref| per tensor (fp64 reference).
TAU = {"f32": 1e-4, "bf16": 2e-2}
TAU_GATES = 1e-4


def dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """Host array -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array; bf16 comes back as uint16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def widen(a: np.ndarray) -> np.ndarray:
    """Exact widening of a downloaded fp32 / bf16-bits array to fp64."""
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    g = widen(gpu) if gpu.dtype in (np.uint16, np.float32) else gpu
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    if scale == 0.0:
        return err
    return err / scale


def assert_close(name, gpu, ref, tau):
    e = rel_err(gpu, ref)
    assert np.isfinite(widen(gpu) if gpu.dtype != np.float64 else gpu).all(), f"{name}: non-finite"
    assert e <= tau, f"{name}: max|err|/max|ref| = {e:.3e} > {tau:.1e}"
    return e


class DevInputs:
    def __init__(self, w: synth.Workload, inp: dict, place: np.ndarray | None = None):
        self.w = w
        self.logits = dev(inp["logits"])
        self.x = dev(inp["x"])
        self.place = dev(inp["place"] if place is None else place)
        self.w_gate = dev(inp["w_gate"])
        self.w_up = dev(inp["w_up"])
        self.w_down = dev(inp["w_down"])


def run_layer(w: synth.Workload, d_in: DevInputs, place=None) -> dict:
    """One pass of the whole HIP path; every output downloaded."""
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    lay = ops.Layer(w.T, w.d, w.E, w.k, w.F, w.G, dt, "cuda", w.n_groups, w.topk_groups)
    pl = d_in.place if place is None else place
    lay.forward(d_in.logits, d_in.x, pl, d_in.w_gate, d_in.w_up, d_in.w_down)
    torch.cuda.synchronize()
    R = int(lay.lay["rank_off"][w.G].item())
    S = int(lay.lay["expert_off"][w.E].item())
    return dict(
        topk_idx=host(lay.topk_idx), gates=host(lay.gates), coact=host(lay.coact),
        rank_mask=host(lay.lay["rank_mask"]).view(np.uint32), rank_off=host(lay.lay["rank_off"]),
        disp_token=host(lay.lay["disp_token"][:R]), expert_off=host(lay.lay["expert_off"]),
        perm_row=host(lay.lay["perm_row"][:S]), slot_of=host(lay.lay["slot_of"]),
        x_disp=host(lay.lay["x_disp"][:R]), h=host(lay.h[:S]), y=host(lay.y[:S]),
        out=host(lay.out), R=R, S=S)


EXACT = ("topk_idx", "coact", "rank_mask", "rank_off", "disp_token", "expert_off", "perm_row",
         "slot_of")


def compare_exact(g: dict, r: dict, keys=EXACT):
    for key in keys:
        a, b = np.asarray(g[key]), np.asarray(r[key])
        if key == "coact":
            b = b.astype(np.int64)
            a = a.astype(np.int64)
        assert a.shape == b.shape, f"{key}: shape {a.shape} vs {b.shape}"
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{key}: {len(bad)} mismatches, first at {bad[0].tolist()}: "
                                 f"gpu {a[tuple(bad[0])]} ref {b[tuple(bad[0])]}")
