"""GPU parity of chunked calls with more tiles than the GPU holds at once, so the single-pass
look-back runs over several rounds of workgroups (a tile's predecessors may already have
retired, and anchor tiles carry the chain forward).  Each mode at a size past one round, with
ragged last tiles, against the fp64 oracle element by element:
  * gated with a prior state, in fp16 (tiles of 16, 32, 128 and 256 tokens, long tiles of 1024)
    and in bfloat16;
  * ungated with fp32 output;
  * fp32 inputs on 64-token tiles;
  * the time mix with its xk/xv outputs.
Also repeated calls on one caller workspace, which must give bitwise equal results (fixed fold
order), calls of different shapes on one workspace (the error word must stay put), and two
such calls running at once on two streams with their own workspaces."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import TOL, check_output, check_state, host, note, to_dev, tol_for, torch

LDS_PER_CU = 160 * 1024
_cache = {}


def assert_past_one_round(B, T, C, chunk, lds_bytes):
    # more tiles than any occupancy could hold at once (LDS alone caps workgroups per CU)
    cus = torch().cuda.get_device_properties(0).multi_processor_count
    tiles = B * ((C + 63) // 64) * ((T + chunk - 1) // chunk)
    bound = cus * (LDS_PER_CU // lds_bytes)
    assert tiles > bound, f"{tiles} tiles fit in one round of {bound}"


def forward(case, chunk, out_dtype=None, workspace=None):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    B, T, C = case["B"], case["T"], case["C"]
    odt = {"f32": t.float32, "f16": t.float16, "bf16": t.bfloat16}[out_dtype or case["out_dtype"]]
    y = t.full((B, T, C), float("nan"), dtype=odt, device="cuda:0")
    so = t.full((3, B, C), float("nan"), device="cuda:0")
    note(f"multi-round forward B={B} T={T} C={C} in={case['in_dtype']} out={out_dtype or case['out_dtype']} "
         f"gated={case.get('r') is not None} chunk={chunk} workspace={'caller' if workspace is not None else 'cached'}")
    idt = case["in_dtype"]
    rw.rwkv4_wkv_forward(to_dev(case["k"], idt), to_dev(case["v"], idt), to_dev(case["w"]), to_dev(case["u"]),
                         y=y, state_in=to_dev(case.get("state_in")), state_out=so, r=to_dev(case.get("r"), idt),
                         out_dtype=odt, algo="chunked", chunk_len=chunk, workspace=workspace)
    t.cuda.synchronize()
    return y, so


def test_multi_round_gated_prior():
    case = wi.forward_case(2, 6000, 2048, seed=81, in_dtype="f16", gated=True, prior=True)
    assert_past_one_round(2, 6000, 2048, 128, 3 * 128 * 64 * 2)
    ref = oracle.forward(case)
    y, so = forward(case, 128)
    check_output(host(y), ref, TOL["f16"], "multi-round gated", out_dtype="f16")
    check_state(host(so), ref, "multi-round gated")


@pytest.mark.parametrize("chunk", [256, 1024])
def test_multi_round_long_tiles(chunk):
    """Chunks of 256 tokens (8-wave tiles staged in LDS) and 1024 tokens (long tiles of 128-token
    sub-tiles) past one resident round, with anchors (chains of 79 and 20 tiles) and a ragged
    last tile."""
    case = wi.forward_case(2, 20000, 2048, seed=86, in_dtype="f16", gated=True, prior=True)
    assert_past_one_round(2, 20000, 2048, chunk, 3 * 128 * 64 * 2)
    key = "long tiles"
    if key not in _cache:
        _cache[key] = oracle.forward(case)
    y, so = forward(case, chunk)
    check_output(host(y), _cache[key], TOL["f16"], f"multi-round long tiles chunk={chunk}", out_dtype="f16")
    check_state(host(so), _cache[key], f"multi-round long tiles chunk={chunk}")


@pytest.mark.parametrize("chunk", [16, 32])
def test_multi_round_short_tiles(chunk):
    """Tiles of 16 tokens (two 8-token waves, anchors every 8 tiles) and 32 tokens (four waves)
    past one resident round: chains of 313 and 157 tiles with a ragged last tile."""
    case = wi.forward_case(2, 5000, 1024, seed=87, in_dtype="f16", gated=True, prior=True)
    waves = chunk // 8
    assert_past_one_round(2, 5000, 1024, chunk, 3 * chunk * 64 * 2 + 4 * waves * 64 * 4)
    key = "short tiles"
    if key not in _cache:
        _cache[key] = oracle.forward(case)
    y, so = forward(case, chunk)
    check_output(host(y), _cache[key], TOL["f16"], f"multi-round short tiles chunk={chunk}", out_dtype="f16")
    check_state(host(so), _cache[key], f"multi-round short tiles chunk={chunk}")


def test_multi_round_bf16_gated_prior():
    case = wi.forward_case(2, 5000, 1024, seed=89, in_dtype="bf16", out_dtype="bf16", gated=True, prior=True)
    assert_past_one_round(2, 5000, 1024, 128, 3 * 128 * 64 * 2)
    ref = oracle.forward(case)
    y, so = forward(case, 128)
    check_output(host(y), ref, tol_for("bf16", "bf16"), "multi-round bf16", out_dtype="bf16")
    check_state(host(so), ref, "multi-round bf16")


def test_multi_round_plain_fp32_out():
    case = wi.forward_case(1, 20000, 1536, seed=82, in_dtype="f16", out_dtype="f32", k_sigma=np.sqrt(2.0))
    assert_past_one_round(1, 20000, 1536, 128, 2 * 128 * 64 * 2)
    ref = oracle.forward(case)
    y, so = forward(case, 128)
    check_output(host(y), ref, TOL["f16"], "multi-round plain f16->f32")
    check_state(host(so), ref, "multi-round plain f16->f32")


def test_multi_round_fp32_inputs_64_token_tiles():
    case = wi.forward_case(1, 8000, 1000, seed=83, in_dtype="f32", prior=True)
    assert_past_one_round(1, 8000, 1000, 64, 2 * 64 * 64 * 4)
    ref = oracle.forward(case)
    y, so = forward(case, 64)
    check_output(host(y), ref, TOL["f32"], "multi-round fp32")
    check_state(host(so), ref, "multi-round fp32")


def test_multi_round_timemix_with_xkv():
    import rwkv_wkv_linear_amd as rw
    t = torch()
    B, T, C = 1, 12000, 2560
    case = wi.timemix_case(B, T, C, seed=84, prior=True)
    assert_past_one_round(B, T, C, 128, 3 * 128 * 64 * 2)
    ref = oracle.timemix(case)
    d = {n: to_dev(case[n]) for n in ("x", "x_prev", "mix_k", "mix_v", "mix_r", "k", "v", "w", "u", "state_in")}
    y = t.full((B, T, C), float("nan"), dtype=t.float16, device="cuda:0")
    xk = t.full((B, T, C), float("nan"), dtype=t.float16, device="cuda:0")
    xv = t.full((B, T, C), float("nan"), dtype=t.float16, device="cuda:0")
    xl = t.full((B, C), float("nan"), dtype=t.float16, device="cuda:0")
    so = t.full((3, B, C), float("nan"), device="cuda:0")
    note(f"multi-round timemix B={B} T={T} C={C} chunk=128")
    rw.rwkv4_timemix_fused(d["x"], d["x_prev"], d["mix_k"], d["mix_v"], d["mix_r"], d["k"], d["v"], d["w"], d["u"],
                           y=y, xk_out=xk, xv_out=xv, x_last=xl, state_in=d["state_in"], state_out=so,
                           algo="chunked", chunk_len=128)
    t.cuda.synchronize()
    check_output(host(y), ref, TOL["f16"], "multi-round timemix", out_dtype="f16")
    check_state(host(so), ref, "multi-round timemix")
    assert np.array_equal(host(xl), ref["x_last"])
    # xk, xv: one fp32 mix rounded once to fp16 (half an ulp plus the fp32 operand error)
    x = case["x"].astype(np.float64)
    xs = np.concatenate([case["x_prev"].astype(np.float64)[:, None, :], x[:, :-1, :]], axis=1)
    for name, got in (("xk", xk), ("xv", xv)):
        want = ref[name]
        bound = 0.5 * np.spacing(np.abs(want).astype(np.float16)).astype(np.float64) + 4e-7 * (np.abs(x) + np.abs(xs))
        assert np.max(np.abs(host(got) - want) - bound) <= 0, f"multi-round timemix: {name}"


def test_multi_round_repeated_calls_one_workspace():
    import rwkv_wkv_linear_amd as rw
    t = torch()
    B, T, C = 1, 30000, 1024
    case = wi.forward_case(B, T, C, seed=85, in_dtype="f16", gated=True, prior=True)
    assert_past_one_round(B, T, C, 128, 3 * 128 * 64 * 2)
    ref = oracle.forward(case)
    nbytes = rw.rwkv4_workspace_bytes(B, T, C, 128)
    ws = t.zeros(nbytes, dtype=t.uint8, device="cuda:0")
    outs = []
    for i in range(3):
        y, so = forward(case, 128, workspace=ws)
        outs.append((y, so))
    check_output(host(outs[0][0]), ref, TOL["f16"], "multi-round repeated", out_dtype="f16")
    check_state(host(outs[0][1]), ref, "multi-round repeated")
    for y, so in outs[1:]:
        assert t.equal(y, outs[0][0]) and t.equal(so, outs[0][1]), "multi-round calls differ"


@pytest.mark.parametrize("workspace", ["caller", "cached"])
def test_concurrent_calls_on_two_streams(workspace):
    """Two chunked calls, each past one resident round, enqueued on two streams with nothing
    ordering them: their workgroups share the GPU, and each call's look-back only ever waits for
    its own earlier-dispatched tiles.  Each call has its own workspace: the caller's, or the one
    the library caches per stream when none is passed."""
    import rwkv_wkv_linear_amd as rw
    t = torch()
    cases = [wi.forward_case(1, 16000, 2048, seed=87, in_dtype="f16", gated=True, prior=True),
             wi.forward_case(2, 9000, 1536, seed=88, in_dtype="f16", out_dtype="f32")]
    for c in cases:
        assert_past_one_round(c["B"], c["T"], c["C"], 128, 3 * 128 * 64 * 2)
    refs = [oracle.forward(c) for c in cases]
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    dev_in, outs = [], []
    for c in cases:
        B, T, C = c["B"], c["T"], c["C"]
        d = {n: to_dev(c.get(n), "f16" if n in ("k", "v", "r") else None) for n in ("k", "v", "r", "w", "u", "state_in")}
        ws = (t.zeros(rw.rwkv4_workspace_bytes(B, T, C, 128), dtype=t.uint8, device="cuda:0")
              if workspace == "caller" else None)
        odt = t.float16 if c["out_dtype"] == "f16" else t.float32
        y = t.full((B, T, C), float("nan"), dtype=odt, device="cuda:0")
        so = t.full((3, B, C), float("nan"), device="cuda:0")
        dev_in.append((d, ws)); outs.append((y, so))
    t.cuda.synchronize()
    note(f"concurrent forwards on two streams, {workspace} workspaces")
    for c, (d, ws), (y, so), st in zip(cases, dev_in, outs, streams):
        rw.rwkv4_wkv_forward(d["k"], d["v"], d["w"], d["u"], y=y, state_in=d["state_in"], state_out=so,
                             r=d["r"], out_dtype=y.dtype, algo="chunked", chunk_len=128, workspace=ws,
                             stream=st)
    t.cuda.synchronize()
    for (d, ws), st in zip(dev_in, streams):
        assert rw.rwkv4_lookback_status(ws, stream=st) is False
    for c, ref, (y, so) in zip(cases, refs, outs):
        what = f"concurrent B{c['B']} T{c['T']} C{c['C']} {workspace} workspace"
        check_output(host(y), ref, TOL["f16"], what, out_dtype=c["out_dtype"])
        check_state(host(so), ref, what)
