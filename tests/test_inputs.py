"""Seeded input generator: determinism, rounding and the parameter recipe (CPU only)."""
import math

import numpy as np

import wkv_inputs as wi


def test_same_seed_same_bytes():
    a = wi.forward_case(2, 33, 70, seed=7, in_dtype="f16", gated=True, prior=True)
    b = wi.forward_case(2, 33, 70, seed=7, in_dtype="f16", gated=True, prior=True)
    for key in ("k", "v", "r", "state_in", "w", "u"):
        assert a[key].tobytes() == b[key].tobytes(), key
    c = wi.forward_case(2, 33, 70, seed=8, in_dtype="f16", gated=True, prior=True)
    assert a["k"].tobytes() != c["k"].tobytes()


def test_timemix_and_step_deterministic():
    a = wi.timemix_case(1, 20, 40, seed=3)
    b = wi.timemix_case(1, 20, 40, seed=3)
    for key in ("x", "x_prev", "mix_k", "mix_v", "mix_r", "k", "v"):
        assert a[key].tobytes() == b[key].tobytes(), key
    l0 = wi.step_layer(0, 4, 32, seed=5)
    l0b = wi.step_layer(0, 4, 32, seed=5)
    l1 = wi.step_layer(1, 4, 32, seed=5)
    assert l0["k"].tobytes() == l0b["k"].tobytes()
    assert l0["k"].tobytes() != l1["k"].tobytes()


def test_f16_rounding_is_nearest_even():
    g = wi.rng_for(0, 123)
    ref = g.standard_normal((1, 10, 10))
    got = wi.forward_case(1, 10, 10, seed=123, in_dtype="f16")["k"]
    # numpy rounds fp64 -> fp16 to nearest (ties to even): no value is more than half an ulp away
    err = np.abs(got.astype(np.float64) - ref)
    ulp = np.spacing(np.abs(got)).astype(np.float64)
    assert np.all(err <= 0.5 * ulp + 1e-300)


def test_decay_bonus_recipe():
    w, u = wi.decay_bonus(768)
    assert w.dtype == np.float32 and u.dtype == np.float32
    assert math.isclose(w[0], -math.exp(-5.0), rel_tol=1e-6)
    assert math.isclose(w[-1], -math.exp(3.0), rel_tol=1e-6)
    assert np.all(np.diff(w.astype(np.float64)) <= 0)
    vals = sorted(set(np.round(u.astype(np.float64), 4)))
    assert np.allclose(vals, [math.log(0.3) - 0.5, math.log(0.3), math.log(0.3) + 0.5], atol=1e-4)
    assert math.isclose(u[0], math.log(0.3), rel_tol=1e-6)   # (0+1) % 3 - 1 = 0


def test_prior_state_ranges():
    st = wi.prior_state(wi.rng_for(1), 8, 768)
    assert st.shape == (3, 8, 768) and st.dtype == np.float32
    assert np.all(st[1] >= 0)
    assert np.all(st[2] >= -5) and np.all(st[2] <= 5)


def test_workload_shapes():
    c1 = wi.workload_inputs(1, T=16)
    assert c1["k"].shape == (8, 16, 768) and c1["k"].dtype == np.float16
    assert c1["state_in"].shape == (3, 8, 768)
    c2 = wi.workload_inputs(2, T=8)
    assert c2["x"].shape == (1, 8, 5120) and c2["x_prev"].shape == (1, 5120)
    c4 = wi.workload_inputs(4, T=64)
    assert c4["k"].dtype == np.float16 and c4["out_dtype"] == "f32"
    layers = wi.workload_inputs(3, layers=2, B=4)
    assert len(layers) == 2 and layers[0]["k"].shape == (4, 5120)


def test_bf16_rounding_matches_round_to_nearest_even():
    """bfloat16 inputs are fp32 values with the low 16 bits cleared by round-to-nearest-even:
    equal to torch's fp32 -> bfloat16 conversion, exactly representable, and within half an
    ulp of the fp32 value (8 significand bits: at most 2^-8 relative)."""
    import torch
    g = np.random.default_rng(5)
    a = np.concatenate([g.standard_normal(50000) * 3, g.uniform(-1e6, 1e6, 1000), [0.0, -0.0, 1.0, 1.00390625]])
    b = wi._round_bf16(a)
    assert b.dtype == np.float32
    assert np.all((b.view(np.uint32) & 0xFFFF) == 0)
    f = a.astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(b, ref)
    nz = f != 0
    assert np.max(np.abs(b[nz] - f[nz]) / np.abs(f[nz])) <= 2.0 ** -8
    assert b[-1] == 1.0  # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even
    case = wi.forward_case(2, 8, 16, seed=3, in_dtype="bf16", gated=True)
    for n in ("k", "v", "r"):
        assert case[n].dtype == np.float32 and np.all((case[n].view(np.uint32) & 0xFFFF) == 0)
