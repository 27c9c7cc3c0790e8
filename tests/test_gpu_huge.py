"""GPU parity past 2^31 elements: B1 T524411 C4104 (2.15e9 elements: the element offsets of
the last ~1150 tokens exceed 2^31, and T and C are ragged against every tile), for
rwkv4_wkv_forward (fp16 k ~ N(0, 2), v ~ N(0, 1), fp32 output and final state) and for
rwkv4_timemix_fused (fp16 x, k, v, x_prev; fp16 y and x_last).  The inputs are drawn on the
device (seeded).  Channels are independent, so only the columns of 64 sampled channels (the
first and last of the ragged last channel tile among them) are copied back: the oracle's
recurrence checks every output element of those channels and their final states, and its
direct sums check 240 points among them (tile edges, the last tokens, tokens whose offsets
pass 2^31).  Over the whole output: every element written and none past the end (canary),
and for the ungated forward every y within [min v, max v] (a convex combination of values).
The decode step runs at B262144 C4104, whose state planes put the offsets of the last plane
past 2^31; sampled lanes (the last ones among them) are checked against the oracle's step."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import TOL, canary_ok, check_output, check_state, note, poisoned, torch

B, T, C = 1, 524411, 4104
_cache = {}


def sample_columns():
    g = np.random.default_rng(2024)
    chans = np.unique(np.concatenate([[0, 1, 63, 64, 2047, 4095, 4096, 4100, 4103],
                                      g.choice(C, 64, replace=False)]))[:64]
    t_big = -(-(2 ** 31) // C)  # first token whose row offset passes 2^31
    toks = np.concatenate([[0, 1, 127, 128, 511, 512, 1023, 1024, 65535, 65536, T - 2, T - 1],
                           np.arange(t_big - 4, t_big + 4), g.integers(0, T, 40)])
    pts_t = np.repeat(toks, 4)
    pts_c = g.integers(0, len(chans), pts_t.size)
    return chans, pts_t, pts_c


def columns(t_dev, ci):
    """[1, T, n] float64 host copy of the sampled channels of a [1, T, C] device tensor."""
    return t_dev[0].index_select(1, ci).double().cpu().numpy()[None]


def forward_case():
    if "fwd" not in _cache:
        t = torch()
        note(f"huge forward inputs B{B} T{T} C{C} drawn on the device")
        c = wi.device_forward_case(B, T, C, seed=2024, k_sigma=np.sqrt(2.0))
        chans, pts_t, pts_c = sample_columns()
        ci = t.from_numpy(chans).to("cuda:0")
        sub = dict(B=1, T=T, C=len(chans), w=c["w"][chans], u=c["u"][chans], k=columns(c["k"], ci),
                   v=columns(c["v"], ci), r=None, state_in=None)
        ref = oracle.forward(sub)
        yp, sp = oracle.wkv_points(sub["k"], sub["v"], sub["w"], sub["u"],
                                   (np.zeros(pts_t.size, dtype=np.int64), pts_t, pts_c))
        _cache["fwd"] = dict(c=c, ci=ci, ref=ref, pts=(pts_t, pts_c), yp=yp, sp=sp,
                             vmin=float(c["v"].min()), vmax=float(c["v"].max()))
    return _cache["fwd"]


@pytest.mark.parametrize("algo,chunk", [("auto", 0), ("two_pass", 128), ("chunked", 512), ("chunked", 1024)])
def test_forward_past_2_31_elements(algo, chunk):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    d = forward_case()
    c = d["c"]
    assert B * T * C > 2 ** 31
    y, yfull = poisoned((B, T, C), "f32")
    so = t.full((3, B, C), float("nan"), device="cuda:0")
    note(f"huge forward B{B} T{T} C{C} f16->f32 algo={algo} chunk={chunk}")
    rw.rwkv4_wkv_forward(c["k"], c["v"], t.from_numpy(c["w"]).cuda(), t.from_numpy(c["u"]).cuda(), y=y,
                         state_out=so, algo=algo, chunk_len=chunk)
    t.cuda.synchronize()
    assert canary_ok(yfull, B * T * C), "write past the end of y"
    assert not bool(t.isnan(y).any()), "an output element was not written"
    lo, hi = float(y.min()), float(y.max())
    assert d["vmin"] - 1e-3 <= lo and hi <= d["vmax"] + 1e-3, f"y outside [min v, max v]: {lo} {hi}"
    ys = columns(y, d["ci"])
    check_output(ys, d["ref"], TOL["f16"], f"huge forward {algo}/{chunk}: 64 channels")
    got = ys[0][d["pts"][0], d["pts"][1]]
    err = float(np.max(np.abs(got - d["yp"]) / d["sp"]))
    note(f"huge forward {algo}/{chunk}: direct sums at {got.size} points {err:.3e}")
    assert err <= TOL["f16"], f"huge {algo}/{chunk}: scaled error {err:.3e} > {TOL['f16']:.1e}"
    check_state(so[:, :, d["ci"]].double().cpu().numpy(), d["ref"], f"huge forward {algo}/{chunk}")
    del y, yfull


@pytest.mark.parametrize("algo,chunk", [("auto", 0), ("two_pass", 128)])
def test_timemix_past_2_31_elements(algo, chunk):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    _cache.pop("fwd", None)  # the forward inputs are no longer needed
    note(f"huge time-mix inputs B{B} T{T} C{C} drawn on the device")
    c = wi.device_timemix_case(B, T, C, seed=2025)
    chans, _, _ = sample_columns()
    ci = t.from_numpy(chans).to("cuda:0")
    sub = dict(B=1, T=T, C=len(chans), w=c["w"][chans], u=c["u"][chans], x=columns(c["x"], ci),
               x_prev=c["x_prev"][:, chans].astype(np.float64), mix_k=c["mix_k"][chans],
               mix_v=c["mix_v"][chans], mix_r=c["mix_r"][chans], k=columns(c["k"], ci), v=columns(c["v"], ci))
    ref = oracle.timemix(sub)
    dv = lambda a: t.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    y, yfull = poisoned((B, T, C), "f16")
    xl = t.full((B, C), float("nan"), dtype=t.float16, device="cuda:0")
    so = t.full((3, B, C), float("nan"), device="cuda:0")
    note(f"huge time mix B{B} T{T} C{C} f16 algo={algo} chunk={chunk}")
    rw.rwkv4_timemix_fused(c["x"], dv(c["x_prev"]), dv(c["mix_k"]), dv(c["mix_v"]), dv(c["mix_r"]), c["k"], c["v"],
                           dv(c["w"]), dv(c["u"]), y=y, x_last=xl, state_out=so, algo=algo, chunk_len=chunk)
    t.cuda.synchronize()
    assert canary_ok(yfull, B * T * C), "write past the end of y"
    assert not bool(t.isnan(y).any()), "an output element was not written"
    check_output(columns(y, ci), ref, TOL["f16"], f"huge time mix {algo}/{chunk}: 64 channels", out_dtype="f16")
    check_state(so[:, :, ci].double().cpu().numpy(), ref, f"huge time mix {algo}/{chunk}")
    assert np.array_equal(xl[:, ci].double().cpu().numpy(), ref["x_last"]), "x_last differs"
    del y, yfull, c


def test_step_state_offsets_past_2_31():
    import rwkv_wkv_linear_amd as rw
    t = torch()
    _cache.clear()
    Bs = 262144
    assert 2 * Bs * C > 2 ** 31
    note(f"huge decode layer B{Bs} C{C} drawn on the device")
    lay = wi.device_step_layer(Bs, C, seed=2026)
    g = np.random.default_rng(2026)
    lb = np.concatenate([[0, 0, Bs - 1, Bs - 1, Bs - 1], g.integers(0, Bs, 251)])
    lc = np.concatenate([[0, C - 1, 0, C - 4, C - 1], g.integers(0, C, 251)])
    bi, cj = t.from_numpy(lb).cuda(), t.from_numpy(lc).cuda()
    pick = lambda a: a[bi, cj].double().cpu().numpy()[None]  # noqa: E731  [1, n] lanes as channels
    sub = dict(B=1, C=lb.size, w=lay["w"][lc], u=lay["u"][lc], k=pick(lay["k"]), v=pick(lay["v"]),
               r=pick(lay["r"]), state=np.stack([pick(lay["state"][q]) for q in range(3)]))
    ref = oracle.step(sub)
    y, yfull = poisoned((Bs, C), "f16")
    note(f"huge decode step B{Bs} C{C}")
    rw.rwkv4_wkv_step(lay["k"], lay["v"], lay["r"], t.from_numpy(lay["w"]).cuda(), t.from_numpy(lay["u"]).cuda(),
                      lay["state"], y=y)
    t.cuda.synchronize()
    assert canary_ok(yfull, Bs * C), "write past the end of y"
    assert not bool(t.isnan(y).any()), "an output element was not written"
    check_output(pick(y), ref, TOL["f16"], "huge decode step: sampled lanes", argmax=False, out_dtype="f16")
    check_state(np.stack([pick(lay["state"][q]) for q in range(3)]), ref, "huge decode step: sampled lanes")
    del y, yfull, lay
