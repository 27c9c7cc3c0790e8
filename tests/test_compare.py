"""Known-answer tests of the comparison metrics (oracle/compare.py), CPU only.

The parity gate is only as strict as these metrics, so each is checked against values fixed by
hand: a rescaled state triple reads 0, a perturbation of known size reads that size, the argmax
tie band accepts exactly the rows within tol * S of the top, and the fp16 floor replaces a
yardstick below fp16's smallest normal (2^-14).  The checks are plain functions so that the
mutation test at the end can run them against deliberately wrong copies of the metrics."""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import compare as cmp


def _near(a, b, tol, what):
    assert abs(a - b) <= tol, f"{what}: got {a!r}, expected {b!r}"


def kat_state_rescaled_reads_zero():
    # (aa e^d, bb e^d, pp - d) is the same state as (aa, bb, pp)
    ref = np.array([[1.5, -0.25], [2.0, 0.5], [3.0, -7.0]])
    d = np.array([4.0, -30.0])
    got = np.stack([ref[0] * np.exp(d), ref[1] * np.exp(d), ref[2] - d])
    ea, eb = cmp.state_error(got, ref, np.abs(ref[0]))
    assert ea <= 1e-15 and eb <= 1e-15, (ea, eb)


def kat_state_perturbation_reads_its_size():
    ref = np.array([[1.5, -0.25], [2.0, 0.5], [3.0, -7.0]])
    abs_ref = np.array([3.0, 0.5])  # the |aa| accumulator scale
    got = ref.copy()
    got[1, 1] *= 1 + 1e-4            # bb relative error 1e-4
    got[0, 0] += 2e-5 * abs_ref[0]  # aa error 2e-5 of its scale
    ea, eb = cmp.state_error(got, ref, abs_ref)
    _near(ea, 2e-5, 1e-12, "aa error")
    _near(eb, 1e-4, 1e-12, "bb error")
    # the same perturbation seen through a rescaled triple
    d = np.array([10.0, -3.0])
    got2 = np.stack([got[0] * np.exp(d), got[1] * np.exp(d), got[2] - d])
    ea2, eb2 = cmp.state_error(got2, ref, abs_ref)
    _near(ea2, 2e-5, 1e-11, "aa error, rescaled")
    _near(eb2, 1e-4, 1e-11, "bb error, rescaled")


def kat_state_nonfinite_fails():
    ref = np.array([[1.0], [1.0], [0.0]])
    for bad in (np.array([[np.nan], [1.0], [0.0]]), np.array([[1.0], [np.inf], [0.0]]),
                np.array([[1.0], [1.0], [np.nan]])):
        assert cmp.state_error(bad, ref, np.ones(1)) == (float("inf"), float("inf"))


def kat_scaled_error():
    y_ref = np.array([0.5, -0.25, 1e-6])
    s = np.array([1.0, 0.5, 2.0])
    y = y_ref + np.array([1e-6, -2e-6, 0.0])
    _near(cmp.scaled_error(y, y_ref, s), 4e-6, 1e-15, "scaled error")
    assert cmp.scaled_error(np.array([np.nan, 0, 0]), y_ref, s) == float("inf")
    assert cmp.scaled_error(np.array([0.5, np.inf, 0]), y_ref, s) == float("inf")


def kat_fp16_floor():
    # a yardstick below 2^-14 is raised to 2^-14; above it, it is used as it is
    y_ref = np.array([1e-6, 0.5])
    s = np.array([2e-6, 1.0])
    y = y_ref + np.array([2.0 ** -24, 0.0])  # one fp16 subnormal step on the tiny element
    _near(cmp.scaled_error(y, y_ref, s, cmp.FLOOR["f16"]), 2.0 ** -10, 1e-18, "floored error")
    _near(cmp.scaled_error(y, y_ref, s), 2.0 ** -24 / 2e-6, 1e-12, "unfloored error")
    assert cmp.FLOOR["f16"] == 2.0 ** -14 and cmp.FLOOR["f32"] == 0.0 and cmp.FLOOR["bf16"] == 0.0
    y2 = np.array([1e-6, 0.5 + 1e-4])
    _near(cmp.scaled_error(y2, y_ref, s, cmp.FLOOR["f16"]), 1e-4, 1e-15, "floor leaves large scales alone")


def kat_argmax_band():
    tol = 1e-3
    s = np.ones((1, 4))
    ref = np.array([[0.1, 0.9, 0.8995, -1.0]])  # top-2 gap 5e-4 < tol: a near tie
    n, bad, near = cmp.argmax_check(np.array([[0.1, 0.8, 0.9, -1.0]]), ref, s, tol)
    assert (n, bad, near) == (1, 0, 1), (n, bad, near)  # index 2 lies inside the band
    ref2 = np.array([[0.1, 0.9, 0.85, -1.0]])            # gap 5e-2: no tie
    assert cmp.argmax_check(np.array([[0.1, 0.8, 0.9, -1.0]]), ref2, s, tol) == (1, 1, 0)
    assert cmp.argmax_check(ref2, ref2, s, tol) == (1, 0, 0)
    # the band is tol * S wide, no wider: a gap of 1.5 tol is a real difference
    ref3 = np.array([[0.1, 0.9, 0.9 - 1.5e-3, -1.0]])
    assert cmp.argmax_check(np.array([[0.1, 0.8, 0.9, -1.0]]), ref3, s, tol) == (1, 1, 0)
    # a near tie accepts only indices inside the band: index 0 is far below the top
    assert cmp.argmax_check(np.array([[2.0, 0.9, 0.8995, -1.0]]), ref, s, tol) == (1, 1, 1)
    # the band scales with S: a tiny S makes the same gap a real difference
    assert cmp.argmax_check(np.array([[0.1, 0.8, 0.9, -1.0]]), ref, s * 1e-3, tol) == (1, 1, 0)
    # rows are taken over the last axis; first index on exact ties (with no band, not near ties)
    y3 = np.array([[[1.0, 1.0, 0.0], [0.0, 2.0, 2.0]]])
    assert cmp.argmax_check(y3, y3, np.ones_like(y3), 0.0) == (2, 0, 0)
    assert cmp.argmax_check(y3[..., ::-1].copy(), y3, np.ones_like(y3), 0.0) == (2, 2, 0)


def kat_min_row_cosine():
    y_ref = np.array([[1.0, 0.0], [0.0, 2.0]])
    y = np.array([[1.0, 1.0], [0.0, 5.0]])
    _near(cmp.min_row_cosine(y, y_ref), 1 / np.sqrt(2.0), 1e-15, "cosine")


ALL_KATS = [kat_state_rescaled_reads_zero, kat_state_perturbation_reads_its_size, kat_state_nonfinite_fails,
            kat_scaled_error, kat_fp16_floor, kat_argmax_band, kat_min_row_cosine]


@pytest.mark.parametrize("kat", ALL_KATS, ids=[k.__name__ for k in ALL_KATS])
def test_known_answer(kat):
    kat()


# (function, name, text in the function, replacement): plausible ways the metrics could be too lax
MUTANTS = [
    ("state_error", "raw aa and bb compared, no rescale", "f = np.exp(s[2] - r[2])", "f = 1.0"),
    ("state_error", "rescaled the wrong way", "f = np.exp(s[2] - r[2])", "f = np.exp(r[2] - s[2])"),
    ("state_error", "bb error relative to the tested value", "np.maximum(np.abs(r[1]), 1e-300)",
     "np.maximum(np.abs(s[1] * f), 1.0)"),
    ("state_error", "NaN pp accepted", "or np.any(np.isnan(s[2]))", "or False"),
    ("scaled_error", "NaN ignored", "if not np.all(np.isfinite(y)):", "if False:"),
    ("scaled_error", "floor ignored", "np.maximum(scale_ref, max(floor, 1e-300))", "np.maximum(scale_ref, 1e-300)"),
    ("scaled_error", "mean instead of max", "float(d.max())", "float(d.mean())"),
    ("argmax_check", "band doubled", "band = tol * np.maximum", "band = 2 * tol * np.maximum"),
    ("argmax_check", "any near-tie index accepted", "(near & (top - yr[rows, got] <= band))", "near"),
    ("argmax_check", "band from the absolute value", "band = tol * np.maximum(sr[rows, ref], sr[rows, got])",
     "band = tol * np.maximum(np.abs(yr[rows, ref]), 1.0)"),
]


@pytest.mark.parametrize("func,name,old,new", MUTANTS, ids=[f"{m[0]}: {m[1]}" for m in MUTANTS])
def test_metric_mutant_is_caught(func, name, old, new):
    orig = getattr(cmp, func)
    src = textwrap.dedent(inspect.getsource(orig))
    assert old in src, f"mutation site for '{name}' not found in compare.{func}"
    ns = {}
    exec(compile(src.replace(old, new, 1), f"<mutant of compare.{func}>", "exec"), vars(cmp), ns)
    setattr(cmp, func, ns[func])
    failed = []
    try:
        for kat in ALL_KATS:
            try:
                kat()
            except AssertionError:
                failed.append(kat.__name__)
    finally:
        setattr(cmp, func, orig)
    assert failed, f"mutant '{func}: {name}' passed every known-answer test"
