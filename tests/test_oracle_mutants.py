"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of oracle/wkv_oracle.c with one plausible mistake (a dropped
term, a wrong index or sign, a transposed operand), compiled with gcc into a
temporary directory.  The pins run against it and at least one must fail.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "wkv_oracle.c")

# (name, text in the source, replacement, replace every occurrence)
MUTANTS = [
    ("decay index off by one",
     "(double)age * w + kl[i * stride]", "(double)(age + 1) * w + kl[i * stride]", False),
    ("newest past token decayed",
     "(age == 0) ? kl[i * stride] :", "(age == 0) ? w + kl[i * stride] :", False),
    ("bonus dropped", "double eb = exp(u + kl[t * stride]);", "double eb = exp(kl[t * stride]);", False),
    ("prior decayed once too often", "decay_pow(t, w) * exp(pp0)", "decay_pow(t + 1, w) * exp(pp0)", False),
    ("prior numerator dropped", "num += f * aa0;", "num += 0.0 * aa0;", False),
    ("value index transposed", "num += e * vl[i * stride];", "num += e * vl[t * stride];", False),
    ("gate sign flipped", "1.0 / (1.0 + exp(-r))", "1.0 / (1.0 + exp(r))", False),
    ("recurrence: bonus in the state", "N = ew * N + ek * vt;", "N = ew * N + eu * ek * vt;", False),
    ("recurrence: denominator not decayed", "D = ew * D + ek;", "D = D + ek;", False),
    ("recurrence: bonus missing from denominator", "const double den = D + eu * ek;",
     "const double den = D + ek;", False),
    ("token shift reads the current token", "x[IDX(b, t - 1, c)]", "x[IDX(b, t, c)]", False),
    ("token shift mix transposed", "mix[c] * x[IDX(b, t, c)] + (1.0 - mix[c]) * xs",
     "(1.0 - mix[c]) * x[IDX(b, t, c)] + mix[c] * xs", False),
    ("state not rescaled by its max", "double e = exp(lw - pmax);", "double e = exp(lw);", False),
    ("state prior decayed one step short", "(double)T * wc + pp0) - pmax", "(double)(T - 1) * wc + pp0) - pmax",
     False),
    ("state newest token decayed", "(age == 0) ? k[IDX(b, i, c)] : (double)age * wc + k[IDX(b, i, c)]",
     "(double)(age + 1) * wc + k[IDX(b, i, c)]", True),
    ("scale uses signed v", "absn += e * fabs(vl[i * stride]);", "absn += e * vl[i * stride];", False),
    ("recurrence scale uses signed v", "A = ew * A + ek * fabs(vt);", "A = ew * A + ek * vt;", False),
    ("layer norm: unbiased variance", "var /= (double)C;", "var /= (double)(C - 1);", False),
    ("layer norm: mean over one value too many", "mean /= (double)C;", "mean /= (double)(C + 1);", False),
    ("layer norm: eps outside the root", "1.0 / sqrt(var + eps)", "1.0 / (sqrt(var) + eps)", False),
    ("layer norm: mean not subtracted", "out[r * C + c] = (xr[c] - mean) * inv", "out[r * C + c] = xr[c] * inv",
     False),
    ("layer norm: weight and bias swapped", "* inv * weight[c] + bias[c]", "* inv * bias[c] + weight[c]", False),
    ("gate: sign flipped", "kv[i] / (1.0 + exp(-r[i]))", "kv[i] / (1.0 + exp(r[i]))", False),
    ("gate: receptance and value swapped", "kv[i] / (1.0 + exp(-r[i]))", "r[i] / (1.0 + exp(-kv[i]))", False),
    ("gate: residual dropped", "y[i] = residual ? residual[i] + g : g;", "y[i] = g;", False),
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new,every", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new, every):
    with open(SRC) as f:
        text = f.read()
    assert old in text, f"mutation site for '{name}' not found in the oracle source"
    text = text.replace(old, new) if every else text.replace(old, new, 1)
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    src = os.path.join(workdir, tag + ".c")
    lib = os.path.join(workdir, "lib" + tag + ".so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", lib,
                           src, "-lm"])
    prev = oracle._use_library(lib)
    failed = []
    try:
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except Exception as e:  # AssertionError or a non-finite result
                failed.append(pin.__name__)
    finally:
        oracle._restore_library(prev)
    assert failed, f"mutant '{name}' passed every pin"


# Planted mistakes in the oracle's Python composition (oracle/__init__.py): each is one edit of a
# function's source, compiled in the module's namespace and swapped in for the original while
# the pins run.  (function, name, text in the function, replacement)
PY_MUTANTS = [
    ("timemix", "receptance taken from xk", "r=xr,", "r=xk,"),
    ("timemix", "xr mixed with mix_k", 'xr = token_shift(x, xp, case["mix_r"])',
     'xr = token_shift(x, xp, case["mix_k"])'),
    ("timemix", "x_prev dropped from the receptance shift", 'xr = token_shift(x, xp,', 'xr = token_shift(x, None,'),
    ("timemix", "x_last from the first row", "_f64(x)[:, -1, :]", "_f64(x)[:, 0, :]"),
    ("timemix", "k and v swapped in the WKV", 'fn(case["k"], case["v"], case["w"], case["u"], r=xr',
     'fn(case["v"], case["k"], case["w"], case["u"], r=xr'),
    ("timemix", "xk output mixed with mix_v", 'xk = token_shift(x, xp, case["mix_k"])',
     'xk = token_shift(x, xp, case["mix_v"])'),
    ("timemix", "xv output unshifted", 'xv = token_shift(x, xp, case["mix_v"])', 'xv = _f64(x)'),
    ("timemix", "state of the gate stream", 'st, ab = wkv_state(case["k"], case["v"]', 'st, ab = wkv_state(case["k"], xr'),
    ("forward", "gate dropped", 'r=case.get("r"),', "r=None,"),
    ("forward", "prior state left out of the state", 'st, ab = wkv_state(case["k"], case["v"], case["w"], state_in=case.get("state_in")',
     'st, ab = wkv_state(case["k"], case["v"], case["w"], state_in=None'),
    ("step", "gate dropped", 'r=r, state_in=layer["state"]', 'r=None, state_in=layer["state"]'),
    ("step", "prior state ignored by the output", 'r=r, state_in=layer["state"]', 'r=r, state_in=None'),
    ("shift_mix", "shift of the raw rows", "token_shift(ln, xp, case[mix])", "token_shift(x, xp, case[mix])"),
    ("shift_mix", "x_last from the raw row", 'out["x_last"] = ln[:, -1, :].copy()', 'out["x_last"] = x[:, -1, :].copy()'),
]


@pytest.mark.parametrize("func,name,old,new", PY_MUTANTS, ids=[f"{m[0]}: {m[1]}" for m in PY_MUTANTS])
def test_composition_mutant_is_caught(func, name, old, new):
    import inspect
    import textwrap
    orig = getattr(oracle, func)
    src = textwrap.dedent(inspect.getsource(orig))
    assert old in src, f"mutation site for '{name}' not found in oracle.{func}"
    ns = {}
    exec(compile(src.replace(old, new, 1), f"<mutant of oracle.{func}>", "exec"), vars(oracle), ns)
    setattr(oracle, func, ns[func])
    failed = []
    try:
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except Exception:
                failed.append(pin.__name__)
    finally:
        setattr(oracle, func, orig)
    assert failed, f"mutant '{func}: {name}' passed every pin"
