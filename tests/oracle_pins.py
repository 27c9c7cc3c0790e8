"""Pins for the fp64 oracle: checks against facts that do not come from the oracle.

Each function raises AssertionError when the oracle disagrees with:
  * the hand-worked examples in tests/golden/hand_worked_t3.json;
  * closed forms (w -> -inf two-term weighting, an impulse's geometric decay,
    a prior state's geometric decay);
  * special cases that reduce to library routines (cumulative mean via
    numpy.cumsum, cumulative softmax-weighted mean via scipy.special.softmax,
    the gate via scipy.special.expit);
  * invariants (constant v, affine equivariance, convexity, shift invariance,
    state carried across a split sequence, canonical state with bb >= 1);
  * the two independent forms inside the oracle (direct sums vs recurrence)
    and a 50-digit mpmath evaluation of the sums (rounding only);
  * for the pre-LN prologue and the channel-mix gate: hand-worked examples
    (tests/golden/layer_norm_shift_gate_hand_worked.json), LayerNorm's closed-form
    moments and invariances, torch's float64 layer_norm, and scipy's expit.

They are plain functions so that the mutation tests can run them against
deliberately wrong builds of the oracle.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit, softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _parse(expr):
    """Evaluate the golden files' tiny expression language: numbers, a/b, ln(a), ln(a/b), -ln(a)
    and c*ln(a) (c a number)."""
    if isinstance(expr, (int, float)):
        return float(expr)
    e = expr.strip()
    sign = 1.0
    if e.startswith("-"):
        sign, e = -1.0, e[1:]
    if "*" in e:
        c, rest = e.split("*", 1)
        return sign * float(c) * _parse(rest)
    if e.startswith("ln(") and e.endswith(")"):
        inner = e[3:-1]
        if "/" in inner:
            a, b = inner.split("/")
            return sign * math.log(float(a) / float(b))
        return sign * math.log(float(inner))
    if "/" in e:
        a, b = e.split("/")
        return sign * float(a) / float(b)
    return sign * float(e)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b) / np.maximum(np.abs(b), 1.0)) if a.size else 0.0
    assert err <= tol, f"{what}: max error {err:.3e} > {tol:.1e}"


def _rand_case(seed, B=2, T=29, C=5, prior=True, gated=True, kscale=1.5):
    g = _rng(seed)
    w = -np.exp(g.uniform(-4, 2, C))
    u = g.uniform(-1.5, 1.0, C)
    k = g.normal(0, kscale, (B, T, C))
    v = g.normal(0, 1, (B, T, C))
    r = g.normal(0, 1, (B, T, C)) if gated else None
    st = None
    if prior:
        st = np.stack([g.normal(0, 1, (B, C)), np.abs(g.normal(0, 1, (B, C))) + 0.05,
                       g.uniform(-3, 3, (B, C))])
    return w, u, k, v, r, st


# ----------------------------------------------------------------------------- golden

def pin_hand_worked():
    with open(os.path.join(GOLDEN, "hand_worked_t3.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        w = np.array([_parse(case["w"])])
        u = np.array([_parse(case["u"])])
        k = np.array([_parse(x) for x in case["k"]]).reshape(1, 3, 1)
        v = np.array(case["v"], dtype=np.float64).reshape(1, 3, 1)
        r = None if case["r"] is None else np.array([_parse(x) for x in case["r"]]).reshape(1, 3, 1)
        st = None
        if case["state_in"] is not None:
            s = case["state_in"]
            st = np.array([_parse(s["aa"]), _parse(s["bb"]), _parse(s["pp"])]).reshape(3, 1, 1)
        want = np.array([_parse(x) for x in case["y"]])
        for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
            y, _ = fn(k, v, w, u, r=r, state_in=st)
            _close(y.ravel(), want, 1e-14, f"hand-worked '{case['name']}' ({fn.__name__})")
        so, _ = oracle.wkv_state(k, v, w, state_in=st)
        exp_state = case["state_out"]
        _close(so.ravel(), [exp_state["aa"], exp_state["bb"], exp_state["pp"]], 1e-14,
               f"hand-worked state '{case['name']}'")
        # the forward's composition (gated WKV and the state after the tokens) on the same case
        out = oracle.forward(dict(k=k, v=v, w=w, u=u, r=r, state_in=st))
        _close(out["y"].ravel(), want, 1e-14, f"hand-worked forward '{case['name']}'")
        _close(out["state"].ravel(), [exp_state["aa"], exp_state["bb"], exp_state["pp"]], 1e-14,
               f"hand-worked forward state '{case['name']}'")
    ts = g["token_shift"]
    x = np.array(ts["x"], dtype=np.float64).reshape(1, 3, 1)
    out = oracle.token_shift(x, np.array([[ts["x_prev"]]], dtype=np.float64),
                             np.array([ts["mix"]]))
    _close(out.ravel(), ts["out"], 1e-15, "hand-worked token shift")


def _golden_timemix():
    with open(os.path.join(GOLDEN, "timemix_hand_worked.json")) as f:
        return json.load(f)


def _grid(rows):
    return np.array([[_parse(e) for e in row] for row in rows], dtype=np.float64)


def pin_timemix_hand_worked():
    """The composition token shift -> r := xr -> gated WKV over the given k, v -> x_last, against
    a case worked by hand (tests/golden/timemix_hand_worked.json), with distinct mix_r, mix_k and
    mix_v so that a mix or a shifted stream taken in the wrong place changes the result."""
    g = _golden_timemix()["timemix"]
    T, C = g["T"], g["C"]
    case = dict(x=_grid(g["x"]).reshape(1, T, C), x_prev=np.array([[_parse(e) for e in g["x_prev"]]]),
                mix_k=np.array(g["mix_k"], float), mix_v=np.array(g["mix_v"], float),
                mix_r=np.array(g["mix_r"], float), k=_grid(g["k"]).reshape(1, T, C),
                v=np.array(g["v"], float).reshape(1, T, C), w=np.array([_parse(e) for e in g["w"]]),
                u=np.array([_parse(e) for e in g["u"]]), state_in=None)
    so = g["state_out"]
    want_state = np.array([[_parse(e) for e in so[f]] for f in ("aa", "bb", "pp")]).reshape(3, 1, C)
    for method in ("recurrence", "direct"):
        out = oracle.timemix(case, method=method)
        _close(out["y"][0], _grid(g["y"]), 1e-14, f"time-mix hand-worked y ({method})")
        for name in ("xr", "xk", "xv"):
            _close(out[name][0], _grid(g[name]), 1e-14, f"time-mix hand-worked {name}")
        _close(out["x_last"][0], [_parse(e) for e in g["x_last"]], 0, "time-mix hand-worked x_last")
        _close(out["state"], want_state, 1e-14, "time-mix hand-worked state")
    # the receptance is the shifted mix itself: ungated WKV times the logistic of xr
    y0, _ = oracle.wkv_direct(case["k"], case["v"], case["w"], case["u"])
    _close(y0[0], _grid(g["wkv"]), 1e-14, "time-mix hand-worked ungated WKV")


def pin_step_hand_worked():
    """One decode token from a prior state (the T = 1 case of the forward), worked by hand."""
    g = _golden_timemix()["step"]
    st = g["state"]
    layer = dict(w=np.array([_parse(g["w"])]), u=np.array([_parse(g["u"])]),
                 k=np.array([[_parse(g["k"])]]), v=np.array([[float(g["v"])]]),
                 r=np.array([[_parse(g["r"])]]),
                 state=np.array([_parse(st["aa"]), _parse(st["bb"]), _parse(st["pp"])]).reshape(3, 1, 1))
    out = oracle.step(layer)
    _close(out["y"].ravel(), [_parse(g["y"])], 1e-15, "step hand-worked y")
    so = g["state_out"]
    _close(out["state"].ravel(), [_parse(so["aa"]), _parse(so["bb"]), _parse(so["pp"])], 1e-15,
           "step hand-worked state")


# ----------------------------------------------------------------------------- closed forms

def pin_full_forgetting():
    """w = -inf: only the newest past token survives, undecayed, beside the bonus term."""
    g = _rng(11)
    B, T, C = 2, 17, 4
    w = np.full(C, -np.inf)
    u = g.uniform(-1, 1, C)
    k = g.normal(0, 1.5, (B, T, C))
    v = g.normal(0, 1, (B, T, C))
    want = np.empty((B, T, C))
    want[:, 0] = v[:, 0]
    a = np.exp(k[:, :-1])
    bo = np.exp(u + k[:, 1:])
    want[:, 1:] = (a * v[:, :-1] + bo * v[:, 1:]) / (a + bo)
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y, _ = fn(k, v, w, u)
        _close(y, want, 1e-13, f"w=-inf closed form ({fn.__name__})")


def pin_impulse_geometric():
    """k = 0, v = impulse at i = 0: y_t = e^{(t-1) w} / (G_t + e^u), G_t = (1 - e^{t w}) / (1 - e^w)."""
    C, T = 3, 40
    w = np.array([-0.05, -0.7, -3.0])
    u = np.array([0.3, -0.4, -1.2])
    k = np.zeros((1, T, C))
    v = np.zeros((1, T, C)); v[0, 0] = 1.0
    t = np.arange(1, T)[:, None]
    G = (1 - np.exp(t * w)) / (1 - np.exp(w))
    want = np.exp((t - 1) * w) / (G + np.exp(u))
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y, _ = fn(k, v, w, u)
        _close(y[0, 1:], want, 1e-13, f"impulse geometric decay ({fn.__name__})")
        _close(y[0, 0], np.ones(C), 1e-15, f"impulse t=0 ({fn.__name__})")


def pin_prior_geometric():
    """v = 0, k = 0, prior (aa0, bb0, pp0): y_t = e^{t w} N0 / (e^{t w} D0 + G_t + e^u)."""
    C, T = 3, 30
    w = np.array([-0.02, -0.5, -2.5])
    u = np.array([-0.3, 0.2, -1.0])
    aa0 = np.array([2.0, -1.5, 0.7]); bb0 = np.array([0.5, 1.2, 3.0]); pp0 = np.array([1.0, -2.0, 0.3])
    st = np.stack([aa0, bb0, pp0]).reshape(3, 1, C)
    k = np.zeros((1, T, C)); v = np.zeros((1, T, C))
    t = np.arange(T)[:, None]
    G = (1 - np.exp(t * w)) / (1 - np.exp(w))
    N0 = aa0 * np.exp(pp0); D0 = bb0 * np.exp(pp0)
    want = np.exp(t * w) * N0 / (np.exp(t * w) * D0 + G + np.exp(u))
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y, _ = fn(k, v, w, u, state_in=st)
        _close(y[0], want, 1e-13, f"prior geometric decay ({fn.__name__})")


# ----------------------------------------------------------------------------- library routines

def pin_cumulative_mean():
    """w = 0, u = 0, k = 0: every past token and the current one weigh 1 -> cumulative mean."""
    g = _rng(5)
    B, T, C = 2, 50, 3
    v = g.normal(0, 1, (B, T, C))
    z = np.zeros(C)
    want = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y, _ = fn(np.zeros((B, T, C)), v, z, z)
        _close(y, want, 1e-13, f"cumulative mean ({fn.__name__})")


def pin_softmax_mean():
    """w = 0: y_t = softmax([k_0 .. k_{t-1}, k_t + u]) . v_{0..t}."""
    g = _rng(6)
    T, C = 25, 3
    k = g.normal(0, 2, (1, T, C)); v = g.normal(0, 1, (1, T, C))
    u = np.array([0.7, -0.9, 0.0]); w = np.zeros(C)
    want = np.empty((T, C))
    for c in range(C):
        for t in range(T):
            logits = k[0, : t + 1, c].copy()
            logits[t] += u[c]
            want[t, c] = softmax(logits) @ v[0, : t + 1, c]
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y, _ = fn(k, v, w, u)
        _close(y[0], want, 1e-13, f"softmax-weighted mean ({fn.__name__})")


def pin_gate_logistic():
    w, u, k, v, r, st = _rand_case(7)
    y0, _ = oracle.wkv_direct(k, v, w, u, state_in=st)
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y, _ = fn(k, v, w, u, r=r, state_in=st)
        _close(y, y0 * expit(r), 1e-13, f"gate = expit ({fn.__name__})")


def pin_token_shift_library():
    g = _rng(8)
    B, T, C = 2, 9, 6
    x = g.normal(0, 1, (B, T, C)); xp = g.normal(0, 1, (B, C)); mix = g.uniform(0, 1, C)
    xs = np.concatenate([xp[:, None, :], x[:, :-1, :]], axis=1)
    _close(oracle.token_shift(x, xp, mix), mix * x + (1 - mix) * xs, 1e-15, "token shift")
    _close(oracle.token_shift(x, xp, np.ones(C)), x, 0, "token shift mix=1")
    _close(oracle.token_shift(x, xp, np.zeros(C)), xs, 0, "token shift mix=0")
    xs0 = np.concatenate([np.zeros((B, 1, C)), x[:, :-1, :]], axis=1)
    _close(oracle.token_shift(x, None, np.zeros(C)), xs0, 0, "token shift, no x_prev")


# ----------------------------------------------------------------------------- invariants

def pin_constant_v():
    g = _rng(9)
    w, u, k, _, _, _ = _rand_case(9, prior=False, gated=False)
    v = np.full_like(k, 1.75)
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y, _ = fn(k, v, w, u)
        _close(y, v, 1e-14, f"constant v, empty state ({fn.__name__})")
        bb0 = np.abs(g.normal(0, 1, (k.shape[0], k.shape[2]))) + 0.1
        st = np.stack([1.75 * bb0, bb0, g.uniform(-3, 3, bb0.shape)])
        y, _ = fn(k, v, w, u, state_in=st)
        _close(y, v, 1e-14, f"constant v, consistent prior ({fn.__name__})")


def pin_affine_equivariance():
    w, u, k, v, _, st = _rand_case(10, gated=False)
    al, be = -2.5, 0.75
    st2 = st.copy(); st2[0] = al * st[0] + be * st[1]
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y1, _ = fn(k, v, w, u, state_in=st)
        y2, _ = fn(k, al * v + be, w, u, state_in=st2)
        _close(y2, al * y1 + be, 1e-12, f"affine equivariance ({fn.__name__})")


def pin_convexity_and_scale():
    w, u, k, v, _, _ = _rand_case(12, prior=False, gated=False)
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y, s = fn(k, v, w, u)
        lo = np.minimum.accumulate(v, axis=1); hi = np.maximum.accumulate(v, axis=1)
        assert np.all(y >= lo - 1e-12) and np.all(y <= hi + 1e-12), "convexity"
        assert np.all(np.abs(y) <= s * (1 + 1e-12)), "|y| <= scale"
        sa, _ = fn(k, np.abs(v), w, u)
        _close(s, sa, 1e-13, f"scale = wkv of |v| ({fn.__name__})")


def pin_shift_invariance():
    w, u, k, v, r, st = _rand_case(13)
    y0, _ = oracle.wkv_direct(k, v, w, u, r=r, state_in=st)
    for d in (-100.0, 100.0):
        st2 = st.copy(); st2[2] = st[2] + d
        for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
            y, _ = fn(k + d, v, w, u, r=r, state_in=st2)
            _close(y, y0, 1e-11, f"shift invariance d={d} ({fn.__name__})")


def pin_state_split_carry():
    w, u, k, v, r, st = _rand_case(14, T=41)
    T1 = 17
    y_full, _ = oracle.wkv_direct(k, v, w, u, r=r, state_in=st)
    s_full, _ = oracle.wkv_state(k, v, w, state_in=st)
    s_mid, _ = oracle.wkv_state(k[:, :T1], v[:, :T1], w, state_in=st)
    for fn in (oracle.wkv_direct, oracle.wkv_recurrence):
        y2, _ = fn(k[:, T1:], v[:, T1:], w, u, r=r[:, T1:], state_in=s_mid)
        _close(y2, y_full[:, T1:], 1e-12, f"split-sequence carry ({fn.__name__})")
    s_end, _ = oracle.wkv_state(k[:, T1:], v[:, T1:], w, state_in=s_mid)
    f = np.exp(s_end[2] - s_full[2])
    _close(s_end[0] * f, s_full[0], 1e-12, "split carry: aa")
    _close(s_end[1] * f, s_full[1], 1e-12, "split carry: bb")
    # one token at a time
    s = st
    for t in range(k.shape[1]):
        s, _ = oracle.wkv_state(k[:, t:t + 1], v[:, t:t + 1], w, state_in=s)
    f = np.exp(s[2] - s_full[2])
    _close(s[0] * f, s_full[0], 1e-12, "token-by-token carry: aa")
    _close(s[1] * f, s_full[1], 1e-12, "token-by-token carry: bb")


def pin_state_canonical():
    """Empty prior: the largest term has weight exactly 1, so 1 <= bb <= T; and pp equals the
    running max p <- max(p + w, k_t) that a max-trick recurrence keeps."""
    w, u, k, v, _, _ = _rand_case(15, prior=False, gated=False, T=33)
    s, _ = oracle.wkv_state(k, v, w)
    T = k.shape[1]
    assert np.all(s[1] >= 1 - 1e-12) and np.all(s[1] <= T + 1e-12), "bb range"
    p = np.full(k.shape[::2], -np.inf)
    for t in range(T):
        p = np.maximum(p + w, k[:, t])
    _close(s[2], p, 1e-13, "pp = running max")
    # the state reproduces the next output: y_T from the state equals the direct sum over T+1
    g = _rng(16)
    k2 = np.concatenate([k, g.normal(0, 1, k[:, :1].shape)], axis=1)
    v2 = np.concatenate([v, g.normal(0, 1, v[:, :1].shape)], axis=1)
    y_all, _ = oracle.wkv_direct(k2, v2, w, u)
    y_next, _ = oracle.wkv_direct(k2[:, T:], v2[:, T:], w, u, state_in=s)
    _close(y_next[:, 0], y_all[:, T], 1e-12, "state -> next output")


# ----------------------------------------------------------------------------- cross-form, precision

def pin_direct_vs_recurrence():
    for seed in (21, 22, 23):
        w, u, k, v, r, st = _rand_case(seed, B=3, T=64, C=7)
        yd, sd = oracle.wkv_direct(k, v, w, u, r=r, state_in=st)
        yr, sr = oracle.wkv_recurrence(k, v, w, u, r=r, state_in=st)
        assert np.max(np.abs(yd - yr) / sd) < 1e-12, "direct vs recurrence"
        _close(sr, sd, 1e-12, "scale direct vs recurrence")


def pin_points_match_direct():
    w, u, k, v, r, st = _rand_case(24, B=2, T=40, C=6)
    yd, sd = oracle.wkv_direct(k, v, w, u, r=r, state_in=st)
    g = _rng(25)
    pts = (g.integers(0, 2, 50), g.integers(0, 40, 50), g.integers(0, 6, 50))
    yp, sp = oracle.wkv_points(k, v, w, u, pts, r=r, state_in=st)
    _close(yp, yd[pts], 0, "points vs direct")
    _close(sp, sd[pts], 0, "points scale vs direct")


def pin_mpmath_precision():
    """50-digit evaluation of the same sums: bounds the oracle's fp64 rounding."""
    import mpmath
    mpmath.mp.dps = 50
    w, u, k, v, r, st = _rand_case(26, B=1, T=24, C=2)
    yd, sd = oracle.wkv_direct(k, v, w, u, r=r, state_in=st)
    yr, _ = oracle.wkv_recurrence(k, v, w, u, r=r, state_in=st)
    mpf, mexp = mpmath.mpf, mpmath.exp
    for c in range(2):
        N0 = mpf(st[0, 0, c]) * mexp(mpf(st[2, 0, c]))
        D0 = mpf(st[1, 0, c]) * mexp(mpf(st[2, 0, c]))
        for t in range(24):
            dec = mexp(t * mpf(w[c]))
            num, den = dec * N0, dec * D0
            for i in range(t):
                e = mexp((t - 1 - i) * mpf(w[c]) + mpf(k[0, i, c]))
                num += e * mpf(v[0, i, c]); den += e
            e = mexp(mpf(u[c]) + mpf(k[0, t, c]))
            num += e * mpf(v[0, t, c]); den += e
            yv = num / den / (1 + mexp(-mpf(r[0, t, c])))
            for got in (yd[0, t, c], yr[0, t, c]):
                assert abs(float(yv - mpf(got))) <= 1e-13 * sd[0, t, c], "mpmath precision"


# ----------------------------------------------------------------------------- pre-LN prologue and gate

def _golden_mix():
    with open(os.path.join(GOLDEN, "layer_norm_shift_gate_hand_worked.json")) as f:
        return json.load(f)


def pin_layer_norm_hand_worked():
    g = _golden_mix()["layer_norm"]
    for case in g["cases"]:
        out = oracle.layer_norm(np.array([case["x"]], dtype=np.float64), g["weight"], g["bias"], case["eps"])
        _close(out[0], case["out"], 1e-14, f"layer norm of {case['x']} (eps {case['eps']})")


def pin_layer_norm_moments():
    # eps = 0, unit weight, zero bias: every row has mean 0 and mean square 1 exactly
    g = _rng(21)
    x = g.normal(0, 1, (7, 53)) * g.uniform(0.1, 30, (7, 1)) + g.normal(0, 50, (7, 1))
    z = oracle.layer_norm(x, np.ones(53), np.zeros(53), 0.0)
    assert np.max(np.abs(z.mean(axis=1))) <= 1e-13, "layer norm: row mean not 0"
    assert np.max(np.abs((z * z).mean(axis=1) - 1.0)) <= 1e-13, "layer norm: row mean square not 1"


def pin_layer_norm_library():
    import torch
    g = _rng(22)
    x = g.normal(0, 1, (3, 5, 37)) * 2.5 + 0.7
    wt, bs = g.normal(1, 0.3, 37), g.normal(0, 0.2, 37)
    for eps in (1e-5, 0.5):
        want = torch.nn.functional.layer_norm(torch.from_numpy(x), (37,), torch.from_numpy(wt),
                                              torch.from_numpy(bs), eps).numpy()
        _close(oracle.layer_norm(x, wt, bs, eps), want, 1e-12, f"layer norm vs torch (eps {eps})")


def pin_layer_norm_invariance():
    # with eps = 0 a row's affine change a*x + b (a > 0) cancels; a sign flip flips z
    g = _rng(23)
    x = g.normal(0, 1, (4, 29))
    wt, bs = g.normal(1, 0.3, 29), g.normal(0, 0.2, 29)
    base = oracle.layer_norm(x, wt, bs, 0.0)
    _close(oracle.layer_norm(3.7 * x - 11.0, wt, bs, 0.0), base, 1e-12, "layer norm: affine invariance")
    z = oracle.layer_norm(x, np.ones(29), np.zeros(29), 0.0)
    _close(oracle.layer_norm(-x, np.ones(29), np.zeros(29), 0.0), -z, 1e-13, "layer norm: odd symmetry")


def pin_shift_mix_hand_worked():
    g = _golden_mix()["shift_mix"]
    x = np.array([g["x"]], dtype=np.float64)
    case = dict(x=x, x_prev=np.array([g["x_prev"]], dtype=np.float64), ln_weight=np.array(g["weight"], float),
                ln_bias=np.array(g["bias"], float), ln_eps=g["eps"], mix_k=np.array(g["mix"], float),
                mix_v=None, mix_r=np.array(g["mix"], float))
    out = oracle.shift_mix(case)
    _close(out["xk"][0], g["out"], 1e-15, "shift-mix hand-worked")
    _close(out["xr"][0], g["out"], 1e-15, "shift-mix hand-worked (xr)")
    _close(out["x_last"][0], g["x_last"], 1e-15, "shift-mix x_last")
    assert "xv" not in out, "shift-mix produced an output with no mix"
    # without LayerNorm the prologue is the bare token shift
    case.update(ln_weight=None, ln_bias=None)
    xs = np.concatenate([case["x_prev"][:, None, :], x[:, :-1, :]], axis=1)
    mix = case["mix_k"]
    _close(oracle.shift_mix(case)["xk"], mix * x + (1 - mix) * xs, 1e-15, "shift-mix without LayerNorm")


def pin_receptance_gate():
    g = _golden_mix()["gate"]
    r = np.array([_parse(e) for e in g["r"]])
    _close(oracle.receptance_gate(r, g["kv"], g["residual"]), g["y"], 1e-15, "gate hand-worked")
    rng = _rng(24)
    r, kv, res = rng.normal(0, 3, 101), rng.normal(0, 1, 101), rng.normal(0, 1, 101)
    _close(oracle.receptance_gate(r, kv, res), res + expit(r) * kv, 1e-14, "gate = residual + expit(r) kv")
    _close(oracle.receptance_gate(r, kv), expit(r) * kv, 1e-14, "gate without residual")


ALL_PINS = [
    pin_hand_worked, pin_full_forgetting, pin_impulse_geometric, pin_prior_geometric,
    pin_cumulative_mean, pin_softmax_mean, pin_gate_logistic, pin_token_shift_library,
    pin_constant_v, pin_affine_equivariance, pin_convexity_and_scale, pin_shift_invariance,
    pin_state_split_carry, pin_state_canonical, pin_direct_vs_recurrence,
    pin_points_match_direct, pin_mpmath_precision, pin_layer_norm_hand_worked,
    pin_layer_norm_moments, pin_layer_norm_library, pin_layer_norm_invariance,
    pin_shift_mix_hand_worked, pin_receptance_gate, pin_timemix_hand_worked, pin_step_hand_worked,
]
