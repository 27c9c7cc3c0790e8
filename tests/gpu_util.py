"""Helpers for the GPU parity tests: host<->device marshalling, poisoned outputs with
canaries, and the comparison gate.  Imported only by tests marked `gpu`."""
from __future__ import annotations

import sys

import numpy as np

from oracle import compare as cmp

# Scaled error bar of the outputs, per input dtype.  The oracle reads the rounded inputs, so a
# 2-byte input costs nothing by itself: bfloat16 inputs take fp16's bar.
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
# A bfloat16 output alone rounds by up to half an ulp, 2^-8 relative (8 significand bits), of
# |y| <= S; its bar is twice that, whatever the input dtype.
OUT_TOL = {"f32": 0.0, "f16": 0.0, "bf16": 8e-3}


def tol_for(in_dtype: str, out_dtype: str) -> float:
    return max(TOL[in_dtype], OUT_TOL[out_dtype])
# The state is fp32 arithmetic on inputs that the oracle reads exactly (the same rounded
# values), and it is never rounded to the I/O dtype, so the input dtype does not enter its error:
# one bar for every input dtype, the fp32 bar.  aa is measured against the oracle's |aa|
# accumulator and bb (a sum of positive weights, no cancellation) against itself.
STATE_TOL = 1e-5
CANARY = 4096                       # elements after each output that must stay untouched
CANARY_VALUE = 1232.0               # exact in fp32, fp16 and bfloat16 (7 significant bits)


def note(msg: str):
    """Name the case before a GPU step (unbuffered, so it survives a lost box)."""
    print(f"[gpu-step] {msg}", file=sys.stdout, flush=True)


def torch():
    import torch as t
    return t


def dev():
    return torch().device("cuda:0")


def to_dev(a, dtype_name=None):
    """numpy -> device tensor; dtype_name "bf16" converts the (bfloat16-valued) float32 data
    to torch.bfloat16, which is exact."""
    if a is None:
        return None
    t = torch().from_numpy(np.ascontiguousarray(a)).to(dev())
    return t.to(tdtype(dtype_name)) if dtype_name == "bf16" else t


_TDT = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def tdtype(name):
    return getattr(torch(), _TDT[name])


def poisoned(shape, dtype_name):
    """Output buffer filled with NaN, followed by CANARY sentinel elements.
    Returns (view of the requested shape, full backing tensor)."""
    t = torch()
    n = int(np.prod(shape))
    full = t.full((n + CANARY,), float("nan"), dtype=tdtype(dtype_name) if isinstance(dtype_name, str)
                  else dtype_name, device=dev())
    full[n:] = CANARY_VALUE
    return full[:n].view(*shape), full


def canary_ok(full, n):
    tail = full[n:].float().cpu().numpy()
    return bool(np.all(tail == CANARY_VALUE))


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_output(y, ref, tol, what, argmax=True, out_dtype="f32"):
    """Gate: scaled error <= tol, no NaN, argmax identical (tie band rule).  With an fp16
    output the yardstick is floored at fp16's smallest normal (see oracle.compare)."""
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output (unwritten element or NaN)"
    rep = cmp.report(y, ref, tol, cmp.FLOOR[out_dtype])
    note(f"{what}: scaled {rep['scaled']:.3e} literal {rep['literal']:.3e} min_cos "
         f"{rep['min_cos']:.12f} argmax_mismatch {rep['argmax_mismatch']}/{rep['argmax_rows']} "
         f"near_ties {rep['near_ties']}")
    assert rep["scaled"] <= tol, f"{what}: scaled error {rep['scaled']:.3e} > {tol:.1e}"
    if argmax:
        assert rep["argmax_mismatch"] == 0, f"{what}: {rep['argmax_mismatch']} argmax rows differ"
    return rep


def check_state(state, ref, what):
    """Gate of a final state (compared canonically, see oracle.compare.state_error)."""
    ea, eb = cmp.state_error(state, ref["state"], ref["state_abs"])
    note(f"{what}: state err aa {ea:.3e} bb {eb:.3e}")
    assert ea <= STATE_TOL and eb <= STATE_TOL, \
        f"{what}: state error aa {ea:.3e} bb {eb:.3e} > {STATE_TOL:.1e}"
