"""Helpers for the GPU parity tests: host<->device marshalling, poisoned outputs with
canaries, and the comparison gate.  Imported only by tests marked `gpu`."""
from __future__ import annotations

import sys

import numpy as np

from oracle import compare as cmp

TOL = {"f32": 1e-5, "f16": 2e-3}   # scaled error bar per input dtype
CANARY = 4096                       # elements after each output that must stay untouched


def note(msg: str):
    """Name the case before a GPU step (unbuffered, so it survives a lost box)."""
    print(f"[gpu-step] {msg}", file=sys.stdout, flush=True)


def torch():
    import torch as t
    return t


def dev():
    return torch().device("cuda:0")


def to_dev(a):
    if a is None:
        return None
    return torch().from_numpy(np.ascontiguousarray(a)).to(dev())


_TDT = {"f32": "float32", "f16": "float16"}


def tdtype(name):
    return getattr(torch(), _TDT[name])


def poisoned(shape, dtype_name):
    """Output buffer filled with NaN, followed by CANARY sentinel elements.
    Returns (view of the requested shape, full backing tensor)."""
    t = torch()
    n = int(np.prod(shape))
    full = t.full((n + CANARY,), float("nan"), dtype=tdtype(dtype_name) if isinstance(dtype_name, str)
                  else dtype_name, device=dev())
    full[n:] = 12345.0
    return full[:n].view(*shape), full


def canary_ok(full, n):
    tail = full[n:].float().cpu().numpy()
    return bool(np.all(tail == 12345.0))


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_output(y, ref, tol, what, argmax=True):
    """Gate: scaled error <= tol, no NaN, argmax identical (tie band rule)."""
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output (unwritten element or NaN)"
    rep = cmp.report(y, ref, tol)
    note(f"{what}: scaled {rep['scaled']:.3e} literal {rep['literal']:.3e} min_cos "
         f"{rep['min_cos']:.12f} argmax_mismatch {rep['argmax_mismatch']}/{rep['argmax_rows']} "
         f"near_ties {rep['near_ties']}")
    assert rep["scaled"] <= tol, f"{what}: scaled error {rep['scaled']:.3e} > {tol:.1e}"
    if argmax:
        assert rep["argmax_mismatch"] == 0, f"{what}: {rep['argmax_mismatch']} argmax rows differ"
    return rep


def check_state(state, ref, tol, what):
    ea, eb = cmp.state_error(state, ref["state"], ref["state_abs"])
    note(f"{what}: state err aa {ea:.3e} bb {eb:.3e}")
    assert ea <= tol and eb <= tol, f"{what}: state error aa {ea:.3e} bb {eb:.3e} > {tol:.1e}"
