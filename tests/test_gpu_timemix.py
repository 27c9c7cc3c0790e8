"""GPU parity of rwkv4_timemix_fused (token shift + WKV + receptance gate) against the
fp64 oracle: the RWKV-4 14B layer shape (B1 T1024 C5120 fp16) at full size, the
optional xk/xv outputs, x_last, a prior state, ragged shapes and T = 0."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import (TOL, canary_ok, check_output, check_state, host, note, poisoned, to_dev,
                      torch)

_cache = {}


def run(case, algo="auto", chunk_len=0, with_xkv=False, with_prev=True, label=""):
    import rwkv_wkv_linear_amd as rw
    B, T, C = case["B"], case["T"], case["C"]
    dt = case["in_dtype"]
    y, yfull = poisoned((B, T, C), case["out_dtype"])
    so, sofull = poisoned((3, B, C), "f32")
    xl, xlfull = poisoned((B, C), dt)
    xk = xv = None
    if with_xkv:
        xk, xkfull = poisoned((B, T, C), dt)
        xv, xvfull = poisoned((B, T, C), dt)
    note(f"timemix {label} B={B} T={T} C={C} {dt}->{case['out_dtype']} algo={algo} chunk={chunk_len} "
         f"xkv={with_xkv} prior={case.get('state_in') is not None}")
    rw.rwkv4_timemix_fused(to_dev(case["x"]), to_dev(case["x_prev"]) if with_prev else None,
                           to_dev(case["mix_k"]), to_dev(case["mix_v"]), to_dev(case["mix_r"]),
                           to_dev(case["k"]), to_dev(case["v"]), to_dev(case["w"]), to_dev(case["u"]),
                           y=y, xk_out=xk, xv_out=xv, x_last=xl, state_in=to_dev(case.get("state_in")),
                           state_out=so, chunk_len=chunk_len, algo=algo)
    torch().cuda.synchronize()
    assert canary_ok(yfull, B * T * C) and canary_ok(sofull, 3 * B * C) and canary_ok(xlfull, B * C)
    out = dict(y=host(y), state=host(so), x_last=host(xl))
    if with_xkv:
        assert canary_ok(xkfull, B * T * C) and canary_ok(xvfull, B * T * C)
        out.update(xk=host(xk), xv=host(xv))
    return out


def check_all(out, ref, case, what, with_xkv):
    tol = TOL[case["in_dtype"]]
    check_output(out["y"], ref, tol, what, out_dtype=case["out_dtype"])
    check_state(out["state"], ref, what)
    assert np.array_equal(out["x_last"], ref["x_last"]), f"{what}: x_last differs"
    if with_xkv:
        # fp32 mix, then one round-to-nearest-even to the I/O dtype: within half an ulp of the
        # fp64 value, plus the fp32 arithmetic error on the operands' magnitude
        x = case["x"].astype(np.float64)
        xp = case["x_prev"].astype(np.float64) if case.get("x_prev") is not None else np.zeros(x[:, 0].shape)
        xs = np.concatenate([xp[:, None, :], x[:, :-1, :]], axis=1)
        io = np.float16 if case["in_dtype"] == "f16" else np.float32
        for name in ("xk", "xv"):
            got, want = out[name], ref[name]
            bound = 0.5 * np.spacing(np.abs(want).astype(io)).astype(np.float64) + 4e-7 * (np.abs(x) + np.abs(xs))
            excess = np.max(np.abs(got - want) - bound)
            note(f"{what}: {name} max |err| - bound = {excess:.3e}")
            assert excess <= 0, f"{what}: {name} off by more than half an ulp"

@pytest.mark.parametrize("algo,chunk", [("sequential", 0), ("chunked", 64), ("chunked", 128), ("two_pass", 64),
                                        ("two_pass", 128), ("chunked", 256), ("chunked", 512), ("chunked", 1024),
                                        ("chunked", 16), ("two_pass", 32), ("two_pass", 256)])
@pytest.mark.parametrize("with_xkv", [False, True])
def test_ragged_prior(algo, chunk, with_xkv):
    case = wi.timemix_case(2, 777, 136, seed=61, prior=True)
    key = "ragged"
    if key not in _cache:
        _cache[key] = oracle.timemix(case)
    out = run(case, algo, chunk, with_xkv, label="ragged")
    check_all(out, _cache[key], case, f"timemix ragged {algo}/{chunk}", with_xkv)


@pytest.mark.parametrize("algo,chunk", [("sequential", 0), ("chunked", 64), ("two_pass", 64), ("chunked", 128),
                                        ("chunked", 256), ("chunked", 32), ("two_pass", 16)])
def test_fp32_odd_channels_no_prev(algo, chunk):
    case = wi.timemix_case(1, 300, 37, seed=62, in_dtype="f32", prior=True)
    nop = dict(case, x_prev=np.zeros_like(case["x_prev"]))
    ref = oracle.timemix(nop)
    out = run(case, algo, chunk, with_xkv=True, with_prev=False, label="fp32 odd C no x_prev")
    check_all(out, ref, nop, f"timemix fp32 C=37 {algo}/{chunk}", True)


@pytest.mark.parametrize("T", [80, 129, 160, 250, 272])
@pytest.mark.parametrize("algo,chunk", [("auto", 0), ("chunked", 64), ("chunked", 128), ("two_pass", 128)])
@pytest.mark.parametrize("with_prev", [True, False])
def test_wave_boundaries(T, algo, chunk, with_prev):
    # Every wave of a tile takes the token before its first (the token shift) itself: from x at
    # t0 - 1, from x_prev at t0 = 0.  These lengths put a wave's first token exactly at T (80 with
    # 16-token waves, 160 with 32-token waves), give a tile's first wave a single token (129),
    # and end on a partial wave after full ones (250, 272), on ragged channels (C = 136).
    case = wi.timemix_case(2, T, 136, seed=64 + T, prior=True)
    if not with_prev:
        case = dict(case, x_prev=np.zeros_like(case["x_prev"]))
    key = ("waves", T, with_prev)
    if key not in _cache:
        _cache[key] = oracle.timemix(case)
    out = run(case, algo, chunk, with_prev=with_prev, label=f"wave boundaries T={T}")
    check_all(out, _cache[key], case, f"timemix T={T} {algo}/{chunk} prev={with_prev}", False)


def test_zero_tokens():
    import rwkv_wkv_linear_amd as rw
    t = torch()
    case = wi.timemix_case(2, 3, 64, seed=63, prior=True)
    x = t.empty((2, 0, 64), dtype=t.float16, device="cuda:0")
    xl = t.full((2, 64), float("nan"), dtype=t.float16, device="cuda:0")
    so = t.full((3, 2, 64), float("nan"), device="cuda:0")
    note("timemix T=0")
    rw.rwkv4_timemix_fused(x, to_dev(case["x_prev"]), to_dev(case["mix_k"]), to_dev(case["mix_v"]),
                           to_dev(case["mix_r"]), x.clone(), x.clone(), to_dev(case["w"]),
                           to_dev(case["u"]), x_last=xl, state_in=to_dev(case["state_in"]), state_out=so)
    t.cuda.synchronize()
    assert np.array_equal(host(xl), case["x_prev"].astype(np.float64))
    assert np.array_equal(host(so), case["state_in"].astype(np.float64))


@pytest.mark.parametrize("algo,chunk", [("auto", 0), ("sequential", 0), ("chunked", 64), ("chunked", 128), ("two_pass", 64),
                                        ("two_pass", 128), ("chunked", 256), ("chunked", 1024), ("chunked", 32),
                                        ("two_pass", 256)])
def test_workload_14b_layer(algo, chunk):
    """B1 T1024 C5120 fp16, token shift from x_prev, r = xr, y = sigmoid(xr) wkv (fp16)."""
    case = wi.workload_inputs(2)
    if "w2" not in _cache:
        ref = oracle.timemix(case)
        g = np.random.default_rng(9)
        pts = (np.zeros(2000, dtype=np.int64), g.integers(0, 1024, 2000), g.integers(0, 5120, 2000))
        yp, sp = oracle.wkv_points(case["k"], case["v"], case["w"], case["u"], pts, r=ref["xr"])
        assert np.max(np.abs(yp - ref["y"][pts]) / sp) < 1e-12
        _cache["w2"] = ref
    out = run(case, algo, chunk, label="rwkv4-14b layer")
    check_all(out, _cache["w2"], case, f"14b layer {algo}/{chunk}", False)


def test_workload_14b_layer_with_xkv():
    case = wi.workload_inputs(2)
    if "w2" not in _cache:
        _cache["w2"] = oracle.timemix(case)
    out = run(case, "auto", 0, with_xkv=True, label="rwkv4-14b layer + xk/xv")
    check_all(out, _cache["w2"], case, "14b layer xk/xv", True)
