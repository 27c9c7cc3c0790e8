"""fp64 CPU oracle for the RWKV-4 WKV time-mixing path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark use
this package.  It shares no code with the GPU library (``rwkv_wkv_linear_amd``)
and never imports it.  The arithmetic lives in ``wkv_oracle.c`` (plain C, fp64,
compiled with gcc -O2 -fopenmp, no fast-math); this module only marshals numpy
arrays and composes the documented steps:

  * ``wkv_direct``      -- every output by the direct sums of the definition
                           (the WKV operator of arXiv 2305.13048, cited by the
                           "RWKV-4 14B" page; described by the TR-2026-0009 port
                           report, Methods and Reproducibility);
  * ``wkv_points``      -- selected outputs by the same sums (any sequence length);
  * ``wkv_recurrence``  -- the numerator/denominator recurrence in fp64 linear space;
  * ``wkv_state``       -- the state after T tokens by its definition;
  * ``token_shift``     -- "mix current and previous token" (TR-2026-0009, Reproducibility);
  * ``timemix``         -- token shift -> WKV -> receptance gate, composed from the above;
  * ``step``            -- one decode token: the T = 1 case of the forward;
  * ``layer_norm``      -- LayerNorm over the channels (the "RWKV-4 14B" page, Facts table:
                           LayerNorm before each mixer; the port report's Abstract: pre-LN);
  * ``shift_mix``       -- the pre-LN token-shift prologue of either mixer, composed from
                           ``layer_norm`` and ``token_shift``;
  * ``receptance_gate`` -- channel mixing's gate and residual add (the port report's
                           "channel-mix gating"; the 14B page's channel-mix receptance).

All inputs are converted exactly to float64 (fp16/fp32 values are exact in fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_wkv.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile wkv_oracle.c into liboracle_wkv.so (gcc, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            lib.oracle_wkv_direct.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp,
                                              _dp, _dp, ctypes.c_int]
            lib.oracle_wkv_points.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp,
                                              _i64, _lp, _lp, _lp, _dp, _dp, ctypes.c_int]
            lib.oracle_wkv_state.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp,
                                             ctypes.c_int]
            lib.oracle_wkv_recurrence.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp,
                                                  _dp, _dp, _dp, ctypes.c_int]
            lib.oracle_token_shift.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp]
            lib.oracle_token_shift.restype = None
            lib.oracle_layer_norm.argtypes = [_i64, _i64, _dp, _dp, _dp, ctypes.c_double, _dp]
            lib.oracle_layer_norm.restype = None
            lib.oracle_receptance_gate.argtypes = [_i64, _dp, _dp, _dp, _dp]
            lib.oracle_receptance_gate.restype = None
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_num_threads.restype = None
            _lib = lib
    return _lib


def _use_library(path):
    """Swap the loaded oracle library for the one at `path` (None: the default build).
    Used by the mutation tests, which compile deliberately wrong copies of the
    oracle and check that the pins reject them.  Returns the previous handle."""
    global _lib
    prev = _lib
    with _lock:
        _lib = None
    if path is not None:
        global _LIB
        saved = _LIB
        _LIB = path
        try:
            _load()
        finally:
            _LIB = saved
    return prev


def _restore_library(handle):
    global _lib
    with _lock:
        _lib = handle


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_threads(n: int) -> None:
    """OpenMP threads of the routines that take no thread count (layer_norm, receptance_gate)."""
    _load().oracle_set_num_threads(int(n))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _check(rc, what):
    if rc != 0:
        raise FloatingPointError(f"oracle {what}: non-finite result (inputs out of fp64 range)")


def _shape3(k):
    if k.ndim != 3:
        raise ValueError("activations must be [B, T, C]")
    return k.shape


def wkv_direct(k, v, w, u, r=None, state_in=None, nthreads=0):
    """(y, scale) [B, T, C] float64 by the direct sums.  O(T^2) per channel."""
    k, v, w, u, r, st = map(_f64, (k, v, w, u, r, state_in))
    B, T, C = _shape3(k)
    y = np.empty((B, T, C)); s = np.empty((B, T, C))
    rc = _load().oracle_wkv_direct(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                   _ptr(st), _ptr(y), _ptr(s), nthreads)
    _check(rc, "wkv_direct")
    return y, s


def wkv_points(k, v, w, u, pts, r=None, state_in=None, nthreads=0):
    """(y, scale) at points pts = (b_idx, t_idx, c_idx) by the direct sums."""
    k, v, w, u, r, st = map(_f64, (k, v, w, u, r, state_in))
    B, T, C = _shape3(k)
    pb, pt, pc = (np.ascontiguousarray(p, dtype=np.int64) for p in pts)
    n = pb.size
    if not (pb.size == pt.size == pc.size):
        raise ValueError("point index arrays differ in length")
    if n and (pb.min() < 0 or pb.max() >= B or pt.min() < 0 or pt.max() >= T
              or pc.min() < 0 or pc.max() >= C):
        raise IndexError("point out of range")
    y = np.empty(n); s = np.empty(n)
    rc = _load().oracle_wkv_points(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                   _ptr(st), n, pb.ctypes.data_as(_lp), pt.ctypes.data_as(_lp),
                                   pc.ctypes.data_as(_lp), _ptr(y), _ptr(s), nthreads)
    _check(rc, "wkv_points")
    return y, s


def wkv_recurrence(k, v, w, u, r=None, state_in=None, nthreads=0):
    """(y, scale) [B, T, C] float64 by the fp64 linear-space recurrence.  O(T) per channel."""
    k, v, w, u, r, st = map(_f64, (k, v, w, u, r, state_in))
    B, T, C = _shape3(k)
    y = np.empty((B, T, C)); s = np.empty((B, T, C))
    rc = _load().oracle_wkv_recurrence(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                       _ptr(st), _ptr(y), _ptr(s), nthreads)
    _check(rc, "wkv_recurrence")
    return y, s


def wkv_state(k, v, w, state_in=None, nthreads=0):
    """(state [3, B, C], |aa| scale [B, C]) after all T tokens, by definition."""
    k, v, w, st = map(_f64, (k, v, w, state_in))
    B, T, C = _shape3(k)
    out = np.empty((3, B, C)); ab = np.empty((B, C))
    rc = _load().oracle_wkv_state(B, T, C, _ptr(w), _ptr(k), _ptr(v), _ptr(st), _ptr(out),
                                  _ptr(ab), nthreads)
    _check(rc, "wkv_state")
    return out, ab


def token_shift(x, x_prev, mix):
    """mix * x_t + (1 - mix) * x_{t-1}, with x_{-1} = x_prev (zeros if None)."""
    x, xp, mix = _f64(x), _f64(x_prev), _f64(mix)
    B, T, C = _shape3(x)
    out = np.empty((B, T, C))
    _load().oracle_token_shift(B, T, C, _ptr(x), _ptr(xp), _ptr(mix), _ptr(out))
    return out


def forward(case, method="recurrence", nthreads=0):
    """Oracle outputs for an rwkv4_wkv_forward case dict (see wkv_inputs.forward_case).
    Returns dict(y, scale, state, state_abs)."""
    fn = wkv_recurrence if method == "recurrence" else wkv_direct
    y, s = fn(case["k"], case["v"], case["w"], case["u"], r=case.get("r"),
              state_in=case.get("state_in"), nthreads=nthreads)
    st, ab = wkv_state(case["k"], case["v"], case["w"], state_in=case.get("state_in"),
                       nthreads=nthreads)
    return dict(y=y, scale=s, state=st, state_abs=ab)


def timemix(case, method="recurrence", nthreads=0):
    """Oracle outputs for an rwkv4_timemix_fused case dict (see wkv_inputs.timemix_case):
    token shift -> r = xr -> gated WKV over the given k, v.  Returns
    dict(y, scale, state, state_abs, xk, xv, xr, x_last)."""
    x, xp = case["x"], case["x_prev"]
    xr = token_shift(x, xp, case["mix_r"])
    xk = token_shift(x, xp, case["mix_k"])
    xv = token_shift(x, xp, case["mix_v"])
    fn = wkv_recurrence if method == "recurrence" else wkv_direct
    y, s = fn(case["k"], case["v"], case["w"], case["u"], r=xr,
              state_in=case.get("state_in"), nthreads=nthreads)
    st, ab = wkv_state(case["k"], case["v"], case["w"], state_in=case.get("state_in"),
                       nthreads=nthreads)
    x_last = _f64(x)[:, -1, :].copy() if x.shape[1] > 0 else _f64(xp)
    return dict(y=y, scale=s, state=st, state_abs=ab, xk=xk, xv=xv, xr=xr, x_last=x_last)


def step(layer, nthreads=0):
    """Oracle outputs for one decode token (wkv_inputs.step_layer dict): the forward
    with T = 1 from the layer's state.  Returns dict(y, scale, state, state_abs)."""
    k = _f64(layer["k"])[:, None, :]
    v = _f64(layer["v"])[:, None, :]
    r = _f64(layer["r"])[:, None, :] if layer.get("r") is not None else None
    y, s = wkv_direct(k, v, layer["w"], layer["u"], r=r, state_in=layer["state"],
                      nthreads=nthreads)
    st, ab = wkv_state(k, v, layer["w"], state_in=layer["state"], nthreads=nthreads)
    return dict(y=y[:, 0, :], scale=s[:, 0, :], state=st, state_abs=ab)


def layer_norm(x, weight, bias, eps):
    """LayerNorm of every row of x [..., C] over its channels: (x - mean) / sqrt(var + eps)
    with the biased variance, then * weight + bias (per channel, [C])."""
    x = _f64(x)
    C = x.shape[-1]
    rows = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    wt, bs = _f64(weight), _f64(bias)
    out = np.empty(x.shape)
    _load().oracle_layer_norm(rows, C, _ptr(x), _ptr(wt), _ptr(bs), float(eps), _ptr(out))
    return out


def shift_mix(case):
    """Oracle outputs for an rwkv4_shift_mix case dict (see wkv_inputs.shift_mix_case): the row
    LayerNorm when ln_weight is given (else x itself), then the token shift against x_prev (the
    previous token's already normalised row; zeros if None) for each given mix.  Returns dict
    with "ln" [B,T,C], "x_last" [B,C] and "xk", "xv", "xr" for the mixes present."""
    x = _f64(case["x"])
    B, T, C = _shape3(x)
    if case.get("ln_weight") is not None:
        ln = layer_norm(x, case["ln_weight"], case["ln_bias"], case["ln_eps"])
    else:
        ln = x
    out = {"ln": ln}
    xp = case.get("x_prev")
    for name, mix in (("xk", "mix_k"), ("xv", "mix_v"), ("xr", "mix_r")):
        if case.get(mix) is not None:
            out[name] = token_shift(ln, xp, case[mix]) if T > 0 else np.empty((B, 0, C))
    if T > 0:
        out["x_last"] = ln[:, -1, :].copy()
    else:
        out["x_last"] = _f64(xp) if xp is not None else np.zeros((B, C))
    return out


def receptance_gate(r, kv, residual=None):
    """y = residual + kv / (1 + e^{-r}) elementwise (residual None: 0)."""
    r, kv = _f64(r), _f64(kv)
    res = _f64(residual) if residual is not None else None
    y = np.empty(r.shape)
    _load().oracle_receptance_gate(r.size, _ptr(r), _ptr(kv), _ptr(res) if res is not None else None, _ptr(y))
    return y
