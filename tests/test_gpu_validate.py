"""GPU checks of the routing validator (moe_validate_routing) and of the
MOE_DEBUG hook of the binding: clean inputs raise no flag; each planted bad
value (planted on the host, read only by the validator's own in-bounds loads)
raises exactly its flag."""
import numpy as np
import pytest
import torch

from routing_dispatch_expert_top_amd import ops, synth
from tests.gpu_helpers import DevInputs, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()


def _inputs(T=1000, E=64, k=6, G=8, seed=0):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx = np.argsort(-logits, axis=1)[:, :k].astype(np.int32)
    place = (np.arange(E) % G).astype(np.int32)
    return logits, idx, place


def test_clean_inputs_have_no_flags():
    logits, idx, place = _inputs()
    logits[3, :5] = -np.inf  # -inf is a mask, not an error
    assert ops.moe_validate_routing(dev(logits), dev(idx), 64, dev(place), 8) == 0


@pytest.mark.parametrize("what,flag", [("nan", ops.MOE_BAD_LOGIT), ("neg", ops.MOE_BAD_EXPERT),
                                       ("big", ops.MOE_BAD_EXPERT),
                                       ("repeat", ops.MOE_BAD_REPEAT),
                                       ("rank", ops.MOE_BAD_RANK), ("negrank", ops.MOE_BAD_RANK)])
def test_each_planted_value_raises_its_flag(what, flag):
    logits, idx, place = _inputs(seed=1)
    if what == "nan":
        logits[997, 63] = np.nan
    elif what == "neg":
        idx[0, 2] = -1
    elif what == "big":
        idx[999, 5] = 64
    elif what == "repeat":
        idx[500, 4] = idx[500, 1]
    elif what == "rank":
        place[63] = 8
    else:
        place[0] = -3
    assert ops.moe_validate_routing(dev(logits), dev(idx), 64, dev(place), 8) == flag
    # each check can be skipped by passing NULL for its array
    if flag == ops.MOE_BAD_LOGIT:
        assert ops.moe_validate_routing(None, dev(idx), 64, dev(place), 8) == 0


def test_debug_hook_raises_before_dispatch(monkeypatch):
    """With MOE_DEBUG=1, Layer.forward validates after routing and raises on a
    placement rank outside [0,G) before any layout kernel reads it."""
    w = synth.custom(name="dbg", T=256, d=64, E=16, k=4, F=64, G=4, dtype="bf16", clusters=4)
    inp = synth.make(w)
    d_in = DevInputs(w, inp)
    lay = ops.Layer(w.T, w.d, w.E, w.k, w.F, w.G, torch.bfloat16, "cuda")
    monkeypatch.setenv("MOE_DEBUG", "1")
    lay.forward(d_in.logits, d_in.x, d_in.place, d_in.w_gate, d_in.w_up, d_in.w_down)
    bad = inp["place"].copy()
    bad[5] = w.G
    with pytest.raises(ValueError, match="rank outside"):
        lay.forward(d_in.logits, d_in.x, dev(bad), d_in.w_gate, d_in.w_up, d_in.w_down)
