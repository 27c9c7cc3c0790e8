"""GPU checks of the look-back publish policies of the single-pass chunked scan (RWKV4 WKV,
computed per channel by the recurrence of the "RWKV-4" formulation; the tiles exchange their
states through the workspace).  A state may go into the publishing XCD's L2 first and be
written through after the tile's outputs (RWKV_PUBLISH_L2_FIRST), or be written through at
once (RWKV_PUBLISH_WRITE_THROUGH); AUTO picks the first when every tile of a chain runs on one
XCD.  Every policy must give bitwise the same outputs and state (the fold order is fixed), and
those match the fp64 oracle.  L2_FIRST is also forced on layouts whose chains cross XCDs
(channel tiles per batch not a multiple of 8, and a grid past one resident round, whose chains
rotate over the XCDs), where a reader on another XCD sees a state only once it is written
through."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import TOL, check_output, check_state, host, note, to_dev, torch

POLICIES = ("auto", "write_through", "l2_first")


def run_forward(case, policy, chunk=128):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    B, T, C = case["B"], case["T"], case["C"]
    odt = {"f32": t.float32, "f16": t.float16, "bf16": t.bfloat16}[case["out_dtype"]]
    y = t.full((B, T, C), float("nan"), dtype=odt, device="cuda:0")
    so = t.full((3, B, C), float("nan"), device="cuda:0")
    note(f"publish={policy} forward B={B} T={T} C={C} in={case['in_dtype']} gated={case.get('r') is not None} "
         f"chunk={chunk}")
    idt = case["in_dtype"]
    rw.rwkv4_wkv_forward(to_dev(case["k"], idt), to_dev(case["v"], idt), to_dev(case["w"]), to_dev(case["u"]),
                         y=y, state_in=to_dev(case.get("state_in")), state_out=so, r=to_dev(case.get("r"), idt),
                         out_dtype=odt, algo="chunked", chunk_len=chunk, publish=policy)
    t.cuda.synchronize()
    return host(y), host(so)


def run_timemix(case, policy):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    B, T, C = case["B"], case["T"], case["C"]
    d = {n: to_dev(case[n]) for n in ("x", "x_prev", "mix_k", "mix_v", "mix_r", "k", "v", "w", "u")}
    y = t.full((B, T, C), float("nan"), dtype=t.float16, device="cuda:0")
    so = t.full((3, B, C), float("nan"), device="cuda:0")
    note(f"publish={policy} timemix B={B} T={T} C={C} chunk=128")
    rw.rwkv4_timemix_fused(d["x"], d["x_prev"], d["mix_k"], d["mix_v"], d["mix_r"], d["k"], d["v"], d["w"], d["u"],
                           y=y, state_out=so, algo="chunked", chunk_len=128, publish=policy)
    t.cuda.synchronize()
    return host(y), host(so)


def same_bits(a, b):
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("B,T,C,why", [
    (1, 1024, 768, "12 channel tiles: a chain's tiles alternate between two XCDs"),
    (8, 1024, 768, "96 chains: each chain on one XCD (AUTO takes L2 first)"),
    (3, 2000, 1000, "48 chains, ragged channels and last tile"),
])
def test_policies_agree_gated(B, T, C, why):
    case = wi.forward_case(B, T, C, seed=171, in_dtype="f16", gated=True, prior=True)
    ref = oracle.forward(case)
    outs = {p: run_forward(case, p) for p in POLICIES}
    for p in POLICIES:
        check_output(outs[p][0], ref, TOL["f16"], f"publish={p} ({why})", out_dtype="f16")
        check_state(outs[p][1], ref, f"publish={p} ({why})")
    for p in POLICIES[1:]:
        assert same_bits(outs[p][0], outs["auto"][0]) and same_bits(outs[p][1], outs["auto"][1]), (p, why)


def test_policies_agree_timemix_one_xcd_chains():
    case = wi.timemix_case(1, 2048, 1024, seed=172, prior=False)
    ref = oracle.timemix(case)
    outs = {p: run_timemix(case, p) for p in POLICIES}
    for p in POLICIES:
        check_output(outs[p][0], ref, TOL["f16"], f"timemix publish={p}", out_dtype="f16")
        check_state(outs[p][1], ref, f"timemix publish={p}")
    for p in POLICIES[1:]:
        assert same_bits(outs[p][0], outs["auto"][0]) and same_bits(outs[p][1], outs["auto"][1]), p


def test_l2_first_forced_past_one_round():
    # more tiles than the GPU holds at once: chains rotate over the XCDs from tile to tile, so
    # nearly every reader is on another XCD and waits for the write-through
    case = wi.forward_case(2, 6000, 2048, seed=173, in_dtype="f16", gated=True, prior=True)
    ref = oracle.forward(case)
    wt = run_forward(case, "write_through")
    l2 = run_forward(case, "l2_first")
    check_output(l2[0], ref, TOL["f16"], "publish=l2_first past one round", out_dtype="f16")
    check_state(l2[1], ref, "publish=l2_first past one round")
    assert same_bits(l2[0], wt[0]) and same_bits(l2[1], wt[1])
