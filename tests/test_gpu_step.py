"""GPU parity of rwkv4_wkv_step (batched single-token decode, state in place) against
the fp64 oracle: 40 layers x B256 x C5120 fp16 at full size, plus step-by-step
against a forward over the same tokens."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import TOL, canary_ok, check_output, check_state, host, note, poisoned, to_dev, torch


def test_decode_40_layers():
    import rwkv_wkv_linear_amd as rw
    t = torch()
    for l in range(40):
        layer = wi.step_layer(l, 256, 5120)
        ref = oracle.step(layer)
        st = to_dev(layer["state"])
        y, yfull = poisoned((256, 5120), "f16")
        note(f"step layer {l} B=256 C=5120 f16 gated")
        rw.rwkv4_wkv_step(to_dev(layer["k"]), to_dev(layer["v"]), to_dev(layer["r"]), to_dev(layer["w"]),
                          to_dev(layer["u"]), st, y=y)
        t.cuda.synchronize()
        assert canary_ok(yfull, 256 * 5120)
        check_output(host(y), ref, TOL["f16"], f"decode layer {l}", out_dtype="f16")
        check_state(host(st), ref, f"decode layer {l}")


@pytest.mark.parametrize("gated", [False, True])
def test_steps_equal_sequential_forward(gated):
    """T calls of step reproduce a forward over the same T tokens.  Not bitwise: the
    forward carries the running max as (anchor key, age) across tokens, while each step
    call rounds it to pp = key + age * w once when it stores the state."""
    import rwkv_wkv_linear_amd as rw
    t = torch()
    case = wi.forward_case(3, 50, 72, seed=71, in_dtype="f16", gated=gated, prior=True)
    k, v, w, u = (to_dev(case[n]) for n in ("k", "v", "w", "u"))
    r = to_dev(case["r"]) if gated else None
    so = t.empty((3, 3, 72), device="cuda:0")
    note(f"step vs forward gated={gated}")
    yf = rw.rwkv4_wkv_forward(k, v, w, u, state_in=to_dev(case["state_in"]), state_out=so, r=r,
                              algo="sequential")
    st = to_dev(case["state_in"])
    ys = []
    for i in range(50):
        ys.append(rw.rwkv4_wkv_step(k[:, i].contiguous(), v[:, i].contiguous(),
                                    r[:, i].contiguous() if gated else None, w, u, st))
    t.cuda.synchronize()
    ref = oracle.forward(case)
    check_output(host(yf), ref, TOL["f16"], f"forward gated={gated}", out_dtype="f16")
    check_output(host(t.stack(ys, dim=1)), ref, TOL["f16"], f"step chain gated={gated}", out_dtype="f16")
    check_state(host(so), ref, f"forward gated={gated}")
    check_state(host(st), ref, f"step chain gated={gated}")
    # the two fp32 paths agree far inside the fp16 output bar
    d = np.max(np.abs(host(t.stack(ys, dim=1)) - host(yf)) / np.maximum(ref["scale"], 2.0 ** -14))
    note(f"step chain vs forward: {d:.3e}")
    assert d <= 1e-3


def test_step_fp32_ungated_odd_channels():
    import rwkv_wkv_linear_amd as rw
    t = torch()
    layer = wi.step_layer(0, 5, 203, in_dtype="f32")
    layer["r"] = None
    ref = oracle.step(layer)
    st = to_dev(layer["state"])
    y = t.full((5, 203), float("nan"), device="cuda:0")
    note("step fp32 C=203")
    rw.rwkv4_wkv_step(to_dev(layer["k"]), to_dev(layer["v"]), None, to_dev(layer["w"]), to_dev(layer["u"]),
                      st, y=y)
    t.cuda.synchronize()
    check_output(host(y), ref, TOL["f32"], "step fp32 C=203")
    check_state(host(st), ref, "step fp32 C=203")
