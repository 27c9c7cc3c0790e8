"""GPU parity of the bfloat16 I/O path against the fp64 oracle: rwkv4_wkv_forward with
bf16 inputs and/or outputs on every algorithm and tile length, odd channel counts (per-element
loads), rwkv4_timemix_fused at the RWKV-4 14B layer shape with the xk/xv outputs, and
batched decode.  bf16 inputs hold bf16-rounded draws that the oracle reads exactly; the bar is
fp16's for the arithmetic plus twice the bf16 output rounding (gpu_util.tol_for)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import (canary_ok, check_output, check_state, host, note, poisoned, to_dev, tol_for,
                      torch)

_cache = {}


def _dev(a, dt):
    return to_dev(a, dt)


def run_forward(case, algo, chunk):
    import rwkv_wkv_linear_amd as rw
    B, T, C = case["B"], case["T"], case["C"]
    idt, odt = case["in_dtype"], case["out_dtype"]
    y, yfull = poisoned((B, T, C), odt)
    so, sofull = poisoned((3, B, C), "f32")
    note(f"bf16 forward B={B} T={T} C={C} {idt}->{odt} algo={algo} chunk={chunk}")
    rw.rwkv4_wkv_forward(_dev(case["k"], idt), _dev(case["v"], idt), to_dev(case["w"]), to_dev(case["u"]),
                         y=y, state_in=to_dev(case["state_in"]), state_out=so, r=_dev(case["r"], idt),
                         chunk_len=chunk, algo=algo)
    torch().cuda.synchronize()
    assert canary_ok(yfull, B * T * C) and canary_ok(sofull, 3 * B * C)
    return host(y), host(so)


ALGOS = [("sequential", 0), ("chunked", 64), ("chunked", 128), ("two_pass", 128), ("auto", 0), ("chunked", 512),
         ("chunked", 32), ("two_pass", 16)]


@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "bf16"), ("f32", "bf16")])
@pytest.mark.parametrize("algo,chunk", ALGOS)
def test_forward_ragged_gated_prior(in_dt, out_dt, algo, chunk):
    case = wi.forward_case(2, 1000, 200, seed=141, in_dtype=in_dt, out_dtype=out_dt, gated=True, prior=True)
    key = ("ragged", in_dt)
    if key not in _cache:
        _cache[key] = oracle.forward(case)
    y, st = run_forward(case, algo, chunk)
    tol = tol_for(in_dt, out_dt)
    check_output(y, _cache[key], tol, f"bf16 ragged {in_dt}->{out_dt} {algo}/{chunk}", out_dtype=out_dt)
    check_state(st, _cache[key], f"bf16 ragged {in_dt}->{out_dt} {algo}/{chunk}")


@pytest.mark.parametrize("algo,chunk", [("sequential", 0), ("chunked", 128)])
def test_forward_odd_channels(algo, chunk):
    case = wi.forward_case(3, 300, 203, seed=142, in_dtype="bf16", out_dtype="bf16", gated=True, prior=True)
    ref = oracle.forward(case)
    y, st = run_forward(case, algo, chunk)
    check_output(y, ref, tol_for("bf16", "bf16"), f"bf16 C=203 {algo}/{chunk}", out_dtype="bf16")
    check_state(st, ref, f"bf16 C=203 {algo}/{chunk}")


def _bf16_half_ulp(x):
    # bfloat16 keeps fp32's exponent and 8 significand bits: its spacing is fp32's times 2^16
    return 0.5 * np.spacing(np.abs(x).astype(np.float32)).astype(np.float64) * 65536.0


@pytest.mark.parametrize("with_xkv", [False, True])
def test_timemix_14b_layer(with_xkv):
    """The 14B layer shape in bfloat16 (bench launch configuration: automatic algorithm)."""
    import rwkv_wkv_linear_amd as rw
    t = torch()
    case = wi.timemix_case(1, 1024, 5120, seed=143, in_dtype="bf16", out_dtype="bf16", index=2)
    if "tm" not in _cache:
        _cache["tm"] = oracle.timemix(case)
    ref = _cache["tm"]
    B, T, C = 1, 1024, 5120
    y, yfull = poisoned((B, T, C), "bf16")
    so = t.empty((3, B, C), device="cuda:0")
    xl = t.empty((B, C), dtype=t.bfloat16, device="cuda:0")
    xk = t.empty((B, T, C), dtype=t.bfloat16, device="cuda:0") if with_xkv else None
    xv = t.empty((B, T, C), dtype=t.bfloat16, device="cuda:0") if with_xkv else None
    note(f"bf16 timemix B1 T1024 C5120 xkv={with_xkv}")
    rw.rwkv4_timemix_fused(_dev(case["x"], "bf16"), _dev(case["x_prev"], "bf16"), to_dev(case["mix_k"]),
                           to_dev(case["mix_v"]), to_dev(case["mix_r"]), _dev(case["k"], "bf16"),
                           _dev(case["v"], "bf16"), to_dev(case["w"]), to_dev(case["u"]), y=y, xk_out=xk,
                           xv_out=xv, x_last=xl, state_out=so)
    t.cuda.synchronize()
    assert canary_ok(yfull, B * T * C)
    tol = tol_for("bf16", "bf16")
    check_output(host(y), ref, tol, "bf16 timemix 14b", out_dtype="bf16")
    check_state(host(so), ref, "bf16 timemix 14b")
    assert np.array_equal(host(xl), ref["x_last"])
    if with_xkv:
        x = case["x"].astype(np.float64)
        xs = np.concatenate([case["x_prev"].astype(np.float64)[:, None, :], x[:, :-1, :]], axis=1)
        for name, got in (("xk", xk), ("xv", xv)):
            want = ref[name]
            bound = _bf16_half_ulp(want) + 4e-7 * (np.abs(x) + np.abs(xs))
            excess = np.max(np.abs(host(got) - want) - bound)
            note(f"bf16 timemix: {name} max |err| - bound = {excess:.3e}")
            assert excess <= 0, f"bf16 timemix: {name} off by more than half an ulp"


def test_decode_layers():
    import rwkv_wkv_linear_amd as rw
    t = torch()
    for l in range(4):
        layer = wi.step_layer(l, 256, 5120, seed=144, in_dtype="bf16")
        ref = oracle.step(layer)
        st = to_dev(layer["state"])
        y, yfull = poisoned((256, 5120), "bf16")
        note(f"bf16 decode layer {l}")
        rw.rwkv4_wkv_step(_dev(layer["k"], "bf16"), _dev(layer["v"], "bf16"), _dev(layer["r"], "bf16"),
                          to_dev(layer["w"]), to_dev(layer["u"]), st, y=y)
        t.cuda.synchronize()
        assert canary_ok(yfull, 256 * 5120)
        check_output(host(y), ref, tol_for("bf16", "bf16"), f"bf16 decode layer {l}", out_dtype="bf16")
        check_state(host(st), ref, f"bf16 decode layer {l}")


@pytest.mark.parametrize("algo,chunk", [("sequential", 0), ("chunked", 64), ("chunked", 128), ("two_pass", 128)])
def test_timemix_ragged_prior(algo, chunk):
    """Time-mix in bfloat16 with an odd channel count, a prior state and a ragged last tile."""
    import rwkv_wkv_linear_amd as rw
    t = torch()
    case = wi.timemix_case(2, 700, 203, seed=145, in_dtype="bf16", out_dtype="bf16", prior=True)
    if "tmr" not in _cache:
        _cache["tmr"] = oracle.timemix(case)
    ref = _cache["tmr"]
    B, T, C = 2, 700, 203
    y, yfull = poisoned((B, T, C), "bf16")
    so, sofull = poisoned((3, B, C), "f32")
    xl, xlfull = poisoned((B, C), "bf16")
    note(f"bf16 timemix ragged B2 T700 C203 algo={algo} chunk={chunk}")
    rw.rwkv4_timemix_fused(_dev(case["x"], "bf16"), _dev(case["x_prev"], "bf16"), to_dev(case["mix_k"]),
                           to_dev(case["mix_v"]), to_dev(case["mix_r"]), _dev(case["k"], "bf16"),
                           _dev(case["v"], "bf16"), to_dev(case["w"]), to_dev(case["u"]), y=y, x_last=xl,
                           state_in=to_dev(case["state_in"]), state_out=so, chunk_len=chunk, algo=algo)
    t.cuda.synchronize()
    assert canary_ok(yfull, B * T * C) and canary_ok(sofull, 3 * B * C) and canary_ok(xlfull, B * C)
    tol = tol_for("bf16", "bf16")
    check_output(host(y), ref, tol, f"bf16 timemix ragged {algo}/{chunk}", out_dtype="bf16")
    check_state(host(so), ref, f"bf16 timemix ragged {algo}/{chunk}")
    assert np.array_equal(host(xl), ref["x_last"])
