"""GPU parity past 2^31 elements: B1 T524411 C4104, fp16 k ~ N(0, 2) and v ~ N(0, 1), fp32 output
and final state (2.15e9 elements: the element offsets of the last ~1150 tokens exceed 2^31, and
T and C are ragged against every tile).  The inputs are drawn on the device (seeded); channels
are independent, so only the columns of 64 sampled channels are copied back, and the oracle's
direct sums check the outputs at sampled points of those channels (tile edges, the last tokens,
tokens whose offsets pass 2^31) and its final state checks theirs.  Over the whole output: every
element written, none past the end (canary), and every y within [min v, max v] (it is a convex
combination of values)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import STATE_TOL, TOL, canary_ok, check_state, note, poisoned, torch

B, T, C = 1, 524411, 4104
_case = {}


def case():
    if not _case:
        t = torch()
        note(f"huge inputs B{B} T{T} C{C} drawn on the device")
        c = wi.device_forward_case(B, T, C, seed=2024, k_sigma=np.sqrt(2.0))
        g = np.random.default_rng(2024)
        chans = np.unique(np.concatenate([[0, 1, 63, 64, 2047, 4095, 4096, 4100, 4103],
                                          g.choice(C, 64, replace=False)]))[:64]
        ci = t.from_numpy(chans).to("cuda:0")
        ks = c["k"][0].index_select(1, ci).float().cpu().numpy().astype(np.float64)[None]
        vs = c["v"][0].index_select(1, ci).float().cpu().numpy().astype(np.float64)[None]
        w, u = c["w"][chans], c["u"][chans]
        t_big = -(-(2 ** 31) // C)  # first token whose row offset passes 2^31
        toks = np.concatenate([[0, 1, 127, 128, 511, 512, 1023, 1024, 65535, 65536, T - 2, T - 1],
                               np.arange(t_big - 4, t_big + 4), g.integers(0, T, 40)])
        pts_t = np.repeat(toks, 4)
        pts_c = g.integers(0, len(chans), pts_t.size)
        yp, sp = oracle.wkv_points(ks, vs, w, u, (np.zeros(pts_t.size, dtype=np.int64), pts_t, pts_c))
        st, ab = oracle.wkv_state(ks, vs, w)
        _case.update(c=c, chans=chans, ci=ci, pts_t=pts_t, pts_c=pts_c, yp=yp, sp=sp,
                     ref=dict(state=st, state_abs=ab), vmin=float(c["v"].min()), vmax=float(c["v"].max()))
    return _case


@pytest.mark.parametrize("algo,chunk", [("auto", 0), ("two_pass", 128), ("chunked", 512), ("chunked", 1024)])
def test_forward_past_2_31_elements(algo, chunk):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    d = case()
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
    ti = t.from_numpy(d["pts_t"]).cuda()
    cj = d["ci"][t.from_numpy(d["pts_c"]).cuda()]
    got = y[0][ti, cj].double().cpu().numpy()
    err = float(np.max(np.abs(got - d["yp"]) / d["sp"]))
    note(f"huge {algo}/{chunk}: scaled error at {got.size} points {err:.3e}")
    assert err <= TOL["f16"], f"huge {algo}/{chunk}: scaled error {err:.3e} > {TOL['f16']:.1e}"
    check_state(so[:, :, d["ci"]].double().cpu().numpy(), d["ref"], f"huge {algo}/{chunk}")
    del y, yfull
