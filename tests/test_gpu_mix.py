"""GPU parity of the mixers' elementwise prologue and epilogue against the fp64 oracle:
rwkv4_shift_mix (LayerNorm over the channels + token shift, any of xk/xv/xr, x_last) and
rwkv4_channelmix_gate (residual + sigmoid(r) * kv), every dtype, vector and per-element paths,
ragged rows, T = 0 and T = 1, x_last updated in place over x_prev, and the RWKV-4 14B shapes.

Bar, per element: half an ulp of the output dtype at the value (one rounding of the fp32
result) plus an fp32 arithmetic term.  For the prologue the arithmetic term is 1e-5 of the
element's magnitude scale A = |weight| (|x| + |mean| + sigma) / sigma + |bias| of the rows it
mixes (|x| itself without LayerNorm, |x_prev| for the row before the first): the row mean and
variance are fp32 sums over C values, whose rounding is relative to |x| + |mean|, and
normalising divides by sigma.  For the gate it is 2e-6 of |kv sigmoid(r)| + |residual| (an
exponential, a reciprocal, a product and a sum, a few fp32 ulps each)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import canary_ok, host, note, poisoned, tdtype, to_dev, torch


def half_ulp(v, dtype):
    a = np.abs(np.asarray(v, dtype=np.float64))
    if dtype == "f16":
        return 0.5 * np.spacing(a.astype(np.float16)).astype(np.float64)
    sp = np.spacing(a.astype(np.float32)).astype(np.float64)
    return 0.5 * sp * (65536.0 if dtype == "bf16" else 1.0)


def _excess(got, want, dtype, arith):
    """max over elements of |got - want| - bound (<= 0 passes) and its index; also notes the
    largest ratio |got - want| / bound."""
    bound = half_ulp(np.maximum(np.abs(got), np.abs(want)), dtype) + arith
    err = np.abs(got - want)
    ex = err - bound
    if not ex.size:
        return -1.0, ()
    i = np.unravel_index(np.argmax(ex), ex.shape)
    note(f"  worst err/bound {np.max(err / bound):.3f}")
    return float(ex[i]), i


def _row_scale(case):
    """Magnitude scale A [B, T, C] of each normalised element, and A of x_prev [B, C]."""
    x = case["x"].astype(np.float64)
    if case["ln_weight"] is None:
        A = np.abs(x)
    else:
        mean = x.mean(axis=-1, keepdims=True)
        sig = np.sqrt(((x - mean) ** 2).mean(axis=-1, keepdims=True) + case["ln_eps"])
        A = (np.abs(case["ln_weight"]) * (np.abs(x) + np.abs(mean) + sig) / sig + np.abs(case["ln_bias"]))
    xp = case["x_prev"]
    Ap = np.abs(xp.astype(np.float64)) if xp is not None else np.zeros((case["B"], case["C"]))
    return A, Ap


def run_shift(case, in_place=False, offset=0):
    """Run rwkv4_shift_mix on a case; offset > 0 shifts every activation pointer by that many
    elements (misaligned for 16-byte vectors).  Returns dict of host arrays."""
    import rwkv_wkv_linear_amd as rw
    t = torch()
    B, T, C, dt = case["B"], case["T"], case["C"], case["dtype"]

    def dev_act(a, shape):
        if a is None:
            return None
        src = to_dev(np.ascontiguousarray(a).reshape(-1), dt)
        buf = t.empty(src.numel() + offset, dtype=src.dtype, device="cuda:0")
        buf[offset:] = src
        return buf[offset:].view(*shape)

    x = dev_act(case["x"], (B, T, C)) if T > 0 else t.empty((B, 0, C), dtype=tdtype(dt), device="cuda:0")
    xp = dev_act(case["x_prev"], (B, C))
    outs, fulls = {}, {}
    for name, mix in (("xk", "mix_k"), ("xv", "mix_v"), ("xr", "mix_r")):
        if case[mix] is not None:
            full_shape = (B * T * C + offset,)
            o, full = poisoned(full_shape, dt)
            outs[name] = o[offset:].view(B, T, C)
            fulls[name] = full
    if in_place:
        assert xp is not None
        xl, xlfull = xp, None
    else:
        xlo, xlfull = poisoned((B * C + offset,), dt)
        xl = xlo[offset:].view(B, C)
    note(f"shift_mix B={B} T={T} C={C} {dt} ln={case['ln_weight'] is not None} "
         f"mixes={sorted(outs)} prev={case['x_prev'] is not None} in_place={in_place} offset={offset}")
    rw.rwkv4_shift_mix(x, xp, ln_weight=to_dev(case["ln_weight"]), ln_bias=to_dev(case["ln_bias"]),
                       ln_eps=case["ln_eps"], mix_k=to_dev(case["mix_k"]), mix_v=to_dev(case["mix_v"]),
                       mix_r=to_dev(case["mix_r"]), xk=outs.get("xk"), xv=outs.get("xv"), xr=outs.get("xr"),
                       x_last=xl)
    t.cuda.synchronize()
    for name, full in fulls.items():
        assert canary_ok(full, B * T * C + offset), f"{name}: write past the end"
    if xlfull is not None:
        assert canary_ok(xlfull, B * C + offset), "x_last: write past the end"
    res = {name: host(o) for name, o in outs.items()}
    res["x_last"] = host(xl)
    return res


def check_shift(got, case, what):
    ref = oracle.shift_mix(case)
    dt = case["dtype"]
    A, Ap = _row_scale(case)
    Amix = A
    if case["T"] > 0:
        Aprev = np.concatenate([Ap[:, None, :], A[:, :-1, :]], axis=1)
        Amix = np.maximum(A, Aprev)
    for name in ("xk", "xv", "xr"):
        if name in ref:
            assert name in got
            assert np.all(np.isfinite(got[name])), f"{what}: {name} has unwritten or non-finite elements"
            ex, i = _excess(got[name], ref[name], dt, 1e-5 * Amix)
            note(f"{what}: {name} max |err| - bound = {ex:.3e} at {i}")
            assert ex <= 0, f"{what}: {name} off at {i}: got {got[name][i]!r}, want {ref[name][i]!r}"
    arith_last = 1e-5 * (A[:, -1, :] if case["T"] > 0 else Ap)
    ex, i = _excess(got["x_last"], ref["x_last"], dt, arith_last)
    note(f"{what}: x_last max |err| - bound = {ex:.3e}")
    assert ex <= 0, f"{what}: x_last off at {i}"


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ln", [True, False])
@pytest.mark.parametrize("C", [200, 203])
def test_shift_mix_ragged(dt, ln, C):
    case = wi.shift_mix_case(2, 10, C, seed=150, dtype=dt, ln=ln)
    check_shift(run_shift(case), case, f"shift-mix ragged {dt} ln={ln} C={C}")


@pytest.mark.parametrize("mixes", ["kr", "r", "v"])
def test_shift_mix_subsets_no_prev(mixes):
    case = wi.shift_mix_case(3, 7, 64, seed=151, dtype="f16", mixes=mixes, prior=False)
    check_shift(run_shift(case), case, f"shift-mix mixes={mixes} no x_prev")


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_shift_mix_misaligned(dt):
    case = wi.shift_mix_case(2, 9, 256, seed=152, dtype=dt)
    check_shift(run_shift(case, offset=1), case, f"shift-mix misaligned {dt}")


@pytest.mark.parametrize("T", [1, 2, 3, 4, 7, 40])
def test_shift_mix_in_place_state(T):
    # x_last written over x_prev: the outputs must still see the old x_prev
    case = wi.shift_mix_case(3, T, 136, seed=153 + T, dtype="f16")
    check_shift(run_shift(case, in_place=True), case, f"shift-mix in place T={T}")


@pytest.mark.parametrize("prior", [True, False])
def test_shift_mix_no_tokens(prior):
    case = wi.shift_mix_case(2, 0, 48, seed=160, dtype="f16", prior=prior)
    check_shift(run_shift(case), case, f"shift-mix T=0 prior={prior}")


@pytest.mark.parametrize("dt,C", [("f32", 4096), ("f32", 8192), ("f32", 8200), ("f32", 20003), ("f16", 8192),
                                  ("f16", 8200), ("bf16", 8191), ("bf16", 9001)])
def test_shift_mix_wide_rows(dt, C):
    # rows of up to 8192 channels are read once, a thread per 8-channel chunk; wider rows take
    # their statistics in streamed passes merged pairwise: both sides of the boundary, ragged ends
    case = wi.shift_mix_case(1, 5, C, seed=161, dtype=dt)
    check_shift(run_shift(case), case, f"shift-mix wide {dt} C={C}")


def test_shift_mix_large_offset_and_constant_rows():
    case = wi.shift_mix_case(2, 6, 96, seed=162, dtype="f32")
    x = case["x"].astype(np.float64)
    x[0] = 1000.0 + 0.01 * x[0]                     # mean/sigma ~ 1e5 after rounding to fp32
    x[1, 2] = 3.5                                   # a constant row: variance 0, output = bias
    case["x"] = x.astype(np.float32)
    check_shift(run_shift(case), case, "shift-mix offset and constant rows")


def test_shift_mix_14b_time_mix_prologue():
    """ln1 + token shift of the RWKV-4 14B layer (B1 T1024 C5120 fp16, xk, xv, xr)."""
    case = wi.shift_mix_case(1, 1024, 5120, seed=163, dtype="f16")
    check_shift(run_shift(case), case, "shift-mix 14B time-mix prologue")


def test_shift_mix_14b_decode_channel_mix():
    """ln2 + token shift for one decode token of 256 sequences (channel mixing: xk, xr)."""
    case = wi.shift_mix_case(256, 1, 5120, seed=164, dtype="bf16", mixes="kr")
    check_shift(run_shift(case, in_place=True), case, "shift-mix 14B decode channel-mix")


# ----------------------------------------------------------------------------- gate

def run_gate(case, in_place=False, offset=0):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    n, idt, odt = case["n"], case["in_dtype"], case["out_dtype"]

    def dev(a):
        if a is None:
            return None
        src = to_dev(a, idt)
        buf = t.empty(n + offset, dtype=src.dtype, device="cuda:0")
        buf[offset:] = src
        return buf[offset:]

    r, kv, res = dev(case["r"]), dev(case["kv"]), dev(case["residual"])
    if in_place:
        y, yfull = res, None
    else:
        yo, yfull = poisoned((n + offset,), odt)
        y = yo[offset:]
    note(f"gate n={n} {idt}->{odt} residual={res is not None} in_place={in_place} offset={offset}")
    rw.rwkv4_channelmix_gate(r, kv, res, y)
    t.cuda.synchronize()
    if yfull is not None:
        assert canary_ok(yfull, n + offset), "gate: write past the end"
    return host(y)


def check_gate(y, case, what):
    ref = oracle.receptance_gate(case["r"], case["kv"], case["residual"])
    g = np.abs(case["kv"].astype(np.float64)) / (1.0 + np.exp(-case["r"].astype(np.float64)))
    res = np.abs(case["residual"].astype(np.float64)) if case["residual"] is not None else 0.0
    assert np.all(np.isfinite(y)), f"{what}: unwritten or non-finite elements"
    ex, i = _excess(y, ref, case["out_dtype"], 2e-6 * (g + res))
    note(f"{what}: max |err| - bound = {ex:.3e}")
    assert ex <= 0, f"{what}: off at {i}: got {y[i]!r}, want {ref[i]!r}"


@pytest.mark.parametrize("idt,odt", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "f32"),
                                     ("f32", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("n", [1, 7, 4096, 100003])
def test_gate_dtypes_and_sizes(idt, odt, n):
    case = wi.gate_case(n, seed=170 + n % 97, in_dtype=idt, out_dtype=odt)
    check_gate(run_gate(case), case, f"gate {idt}->{odt} n={n}")


def test_gate_no_residual_misaligned():
    case = wi.gate_case(5000, seed=171, in_dtype="f16", residual=False)
    check_gate(run_gate(case, offset=3), case, "gate no residual, misaligned")


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_gate_in_place_residual(dt):
    case = wi.gate_case(65536, seed=172, in_dtype=dt)
    check_gate(run_gate(case, in_place=True), case, f"gate in place {dt}")


def test_gate_14b_channel_mix_layer():
    """The channel-mix output of the RWKV-4 14B layer: B1 T1024 C5120 fp16 with the residual."""
    case = wi.gate_case(1024 * 5120, seed=173, in_dtype="f16")
    check_gate(run_gate(case), case, "gate 14B layer")


def test_negative_controls():
    """The bars are tight enough to see a dropped step: the GPU's LayerNorm output against the
    oracle without LayerNorm, and the gate against the oracle without the residual, must miss
    the bar by more than 100x."""
    case = wi.shift_mix_case(2, 10, 200, seed=180, dtype="f16")
    got = run_shift(case)
    wrong = dict(case, ln_weight=None, ln_bias=None)
    ref = oracle.shift_mix(wrong)
    A, Ap = _row_scale(case)
    bound = half_ulp(ref["xk"], "f16") + 1e-5 * A
    ratio = np.max(np.abs(got["xk"] - ref["xk"]) / bound)
    note(f"negative control, LayerNorm dropped: err/bound {ratio:.1f}")
    assert ratio > 100
    g = wi.gate_case(4096, seed=181, in_dtype="f16")
    y = run_gate(g)
    ref = oracle.receptance_gate(g["r"], g["kv"], None)
    bound = half_ulp(ref, "f16") + 2e-6 * np.abs(ref)
    ratio = np.max(np.abs(y - ref) / bound)
    note(f"negative control, residual dropped: err/bound {ratio:.1f}")
    assert ratio > 100
