"""Seeded synthetic inputs for the RWKV-4 WKV time-mixing path.

This module is shared by the tests, the benchmark and the oracle's tests, and it holds
none of the recurrence's arithmetic: it only draws random arrays, rounds them
to the I/O dtype, and evaluates the per-channel initialisation recipe for the
decay and bonus parameters.

Recipe (all workloads):
  * generator: numpy PCG64 seeded with ``1000 + workload index`` unless a seed
    is given; draws are fp64 and are rounded (round-to-nearest-even) to the I/O
    dtype -- once for fp32 and fp16, via fp32 for bfloat16, which is held in
    float32 arrays -- so both sides of every comparison consume identical values;
  * decay:  time_decay_c = -5 + 8 * (c / (C-1)) ** 1.35,  w_c = -exp(time_decay_c)
  * bonus:  u_c = 0.5 * (((c + 1) mod 3) - 1) + ln(0.3)
    (the initialisation these workloads are specified with; the pages give no
    trained parameters);
  * a random prior state is (aa ~ N(0,1), bb = |N(0,1)|, pp ~ U(-5,5)) in fp32,
    planar [3, B, C]; bb is a sum of positive weights, so its magnitude is drawn.

The five named workloads follow the shapes of the RWKV-4 169m and 14B models
(d_model 768 and 5120, 40 layers, 1K context) and a long-context case at
hidden size 2048 (the RWKV-GLM card's width).

The mixers' elementwise prologue and epilogue (pre-LN token shift, channel-mix receptance
gate) draw their own cases: activations N(0,1) with, for the LayerNorm input, a per-row
offset N(0, 2^2) and scale U(0.5, 4) so the row statistics matter; LayerNorm weight
N(1, 0.25^2) and bias N(0, 0.1^2) in fp32 (the pages give no trained values); eps 1e-5;
mixes U(0,1); the gate's receptance N(0, 2^2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "WORKLOADS", "Workload", "decay_bonus", "forward_case", "timemix_case",
    "step_layer", "prior_state", "workload_inputs", "rng_for", "shift_mix_case", "gate_case",
    "LN_EPS",
]

# LayerNorm epsilon of the prologue cases: the pages give none; 1e-5 is the usual default of
# a LayerNorm layer.
LN_EPS = 1e-5


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str            # "forward" | "timemix" | "step" | "shift" | "gate"
    B: int
    T: int
    C: int
    in_dtype: str        # "f32" | "f16"
    out_dtype: str
    gated: bool = False
    prior: bool = False
    k_sigma: float = 1.0
    layers: int = 1
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    0: Workload(0, "rwkv4-169m wkv forward B1 T1024 C768 fp32", "forward",
                1, 1024, 768, "f32", "f32"),
    1: Workload(1, "rwkv4-169m gated prefill B8 T1024 C768 f16, prior state", "forward",
                8, 1024, 768, "f16", "f16", gated=True, prior=True),
    2: Workload(2, "rwkv4-14b time-mix fused prefill B1 T1024 C5120 f16", "timemix",
                1, 1024, 5120, "f16", "f16", gated=True),
    3: Workload(3, "rwkv4-14b batched decode 40 layers B256 C5120 f16", "step",
                256, 1, 5120, "f16", "f16", gated=True, prior=True, layers=40),
    4: Workload(4, "long-sequence chunked scan B1 T65536 C2048 f16->f32", "forward",
                1, 65536, 2048, "f16", "f32", k_sigma=math.sqrt(2.0)),
    5: Workload(5, "rwkv4-14b time-mix prologue: ln1 + token shift -> xk, xv, xr B1 T1024 C5120 f16",
                "shift", 1, 1024, 5120, "f16", "f16", prior=True),
    6: Workload(6, "rwkv4-14b channel-mix gate + residual B1 T1024 C5120 f16", "gate",
                1, 1024, 5120, "f16", "f16"),
}

_NP = {"f32": np.float32, "f16": np.float16}


def _round_bf16(a) -> np.ndarray:
    """bfloat16 values (fp32's exponent, 8 significand bits) held in a float32 array: the
    fp64 draw is rounded to fp32, then to bfloat16, each to nearest-even (finite inputs)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _as(a, dtype):
    """Round an fp64 array to an I/O dtype: "f32", "f16", or "bf16" (held in float32)."""
    if dtype == "bf16":
        return _round_bf16(a)
    return np.asarray(a).astype(_NP[dtype])


def rng_for(index: int, seed: int | None = None, stream: int | None = None) -> np.random.Generator:
    """PCG64 generator: seed 1000+index by default; `stream` selects an independent
    sub-stream (used per decode layer)."""
    s = (1000 + index) if seed is None else seed
    if stream is None:
        return np.random.Generator(np.random.PCG64(s))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([s, stream])))


def _normal(rng, shape, dtype, sigma=1.0, shift=0.0):
    a = rng.standard_normal(shape)
    if sigma != 1.0:
        a *= sigma
    if shift != 0.0:
        a += shift
    return _as(a, dtype)


def decay_bonus(C: int):
    """Per-channel (w, u) as fp32 arrays of length C (recipe in the module doc)."""
    c = np.arange(C, dtype=np.float64)
    frac = c / (C - 1) if C > 1 else np.zeros_like(c)
    time_decay = -5.0 + 8.0 * frac ** 1.35
    w = -np.exp(time_decay)
    u = 0.5 * (((c + 1) % 3) - 1) + math.log(0.3)
    return w.astype(np.float32), u.astype(np.float32)


def prior_state(rng, B: int, C: int) -> np.ndarray:
    """Random prior state, planar fp32 [3, B, C] = (aa, bb, pp)."""
    aa = rng.standard_normal((B, C))
    bb = np.abs(rng.standard_normal((B, C)))
    pp = rng.uniform(-5.0, 5.0, (B, C))
    return np.stack([aa, bb, pp]).astype(np.float32)


def forward_case(B, T, C, *, seed, in_dtype="f32", out_dtype=None, gated=False,
                 prior=False, k_sigma=1.0, k_shift=0.0, index=0):
    """Inputs for rwkv4_wkv_forward.  Draw order: k, v, [r], [aa, bb, pp]."""
    g = rng_for(index, seed)
    w, u = decay_bonus(C)
    k = _normal(g, (B, T, C), in_dtype, k_sigma, k_shift)
    v = _normal(g, (B, T, C), in_dtype)
    r = _normal(g, (B, T, C), in_dtype) if gated else None
    st = prior_state(g, B, C) if prior else None
    return dict(B=B, T=T, C=C, w=w, u=u, k=k, v=v, r=r, state_in=st,
                in_dtype=in_dtype, out_dtype=out_dtype or in_dtype)


def device_forward_case(B, T, C, *, seed, k_sigma=1.0, device="cuda:0"):
    """Inputs for rwkv4_wkv_forward too large to draw on the host: fp16 k ~ N(0, k_sigma^2) and
    v ~ N(0, 1) drawn on the device by torch's generator seeded with `seed` (fp32 draws rounded
    once to fp16, RNE), w and u by the recipe above.  Whoever checks results copies back the
    rows or columns it needs; both sides read the identical fp16 values."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    k = torch.randn((B, T, C), generator=g, device=device, dtype=torch.float32)
    if k_sigma != 1.0:
        k.mul_(k_sigma)
    k = k.to(torch.float16)
    v = torch.randn((B, T, C), generator=g, device=device, dtype=torch.float32).to(torch.float16)
    w, u = decay_bonus(C)
    return dict(B=B, T=T, C=C, w=w, u=u, k=k, v=v)


def device_timemix_case(B, T, C, *, seed, device="cuda:0"):
    """Inputs for rwkv4_timemix_fused too large to draw on the host: fp16 x, k, v ~ N(0, 1)
    drawn on the device as in device_forward_case (in that order, from one generator seeded with
    `seed`); x_prev, the mixes, w and u on the host as in timemix_case."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    draw = lambda: torch.randn((B, T, C), generator=g, device=device,  # noqa: E731
                               dtype=torch.float32).to(torch.float16)
    x, k, v = draw(), draw(), draw()
    h = rng_for(2, seed)
    w, u = decay_bonus(C)
    x_prev = _normal(h, (B, C), "f16")
    mix_k = h.uniform(0.0, 1.0, C).astype(np.float32)
    mix_v = h.uniform(0.0, 1.0, C).astype(np.float32)
    mix_r = h.uniform(0.0, 1.0, C).astype(np.float32)
    return dict(B=B, T=T, C=C, w=w, u=u, x=x, x_prev=x_prev, mix_k=mix_k, mix_v=mix_v, mix_r=mix_r,
                k=k, v=v)


def device_step_layer(B, C, *, seed, device="cuda:0"):
    """One decode layer too large to draw on the host: fp16 k, v, r ~ N(0, 1) and the state
    (aa ~ N(0, 1), bb = |N(0, 1)|, pp ~ U(-5, 5), fp32), drawn on the device in that order from
    one generator seeded with `seed`; w and u by the recipe above."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    n = lambda: torch.randn((B, C), generator=g, device=device, dtype=torch.float32)  # noqa: E731
    k, v, r = n().to(torch.float16), n().to(torch.float16), n().to(torch.float16)
    aa, bb = n(), n().abs_()
    pp = torch.rand((B, C), generator=g, device=device, dtype=torch.float32).mul_(10.0).sub_(5.0)
    w, u = decay_bonus(C)
    return dict(B=B, C=C, w=w, u=u, k=k, v=v, r=r, state=torch.stack([aa, bb, pp]))


def timemix_case(B, T, C, *, seed, in_dtype="f16", out_dtype=None, index=2, prior=False):
    """Inputs for rwkv4_timemix_fused.
    Draw order: x, x_prev, mix_k, mix_v, mix_r, k, v, [aa, bb, pp]."""
    g = rng_for(index, seed)
    w, u = decay_bonus(C)
    x = _normal(g, (B, T, C), in_dtype)
    x_prev = _normal(g, (B, C), in_dtype)
    mix_k = g.uniform(0.0, 1.0, C).astype(np.float32)
    mix_v = g.uniform(0.0, 1.0, C).astype(np.float32)
    mix_r = g.uniform(0.0, 1.0, C).astype(np.float32)
    k = _normal(g, (B, T, C), in_dtype)
    v = _normal(g, (B, T, C), in_dtype)
    st = prior_state(g, B, C) if prior else None
    return dict(B=B, T=T, C=C, w=w, u=u, x=x, x_prev=x_prev, mix_k=mix_k, mix_v=mix_v,
                mix_r=mix_r, k=k, v=v, state_in=st, in_dtype=in_dtype,
                out_dtype=out_dtype or in_dtype)


def step_layer(layer: int, B: int, C: int, *, seed=None, in_dtype="f16", index=3):
    """One decode layer: k, v, r [B, C] and a random state [3, B, C].
    Each layer draws from its own sub-stream (seed, layer) in the order k, v, r, aa, bb, pp."""
    g = rng_for(index, seed, stream=layer)
    w, u = decay_bonus(C)
    k = _normal(g, (B, C), in_dtype)
    v = _normal(g, (B, C), in_dtype)
    r = _normal(g, (B, C), in_dtype)
    st = prior_state(g, B, C)
    return dict(B=B, C=C, w=w, u=u, k=k, v=v, r=r, state=st, in_dtype=in_dtype)


def workload_inputs(index: int, seed: int | None = None, **shape):
    """Inputs for a named workload; `shape` may override B, T, C for reduced cases."""
    wl = WORKLOADS[index]
    B = shape.get("B", wl.B)
    T = shape.get("T", wl.T)
    C = shape.get("C", wl.C)
    s = (1000 + index) if seed is None else seed
    if wl.kind == "forward":
        return forward_case(B, T, C, seed=s, in_dtype=wl.in_dtype, out_dtype=wl.out_dtype,
                            gated=wl.gated, prior=wl.prior, k_sigma=wl.k_sigma, index=index)
    if wl.kind == "timemix":
        return timemix_case(B, T, C, seed=s, in_dtype=wl.in_dtype, out_dtype=wl.out_dtype,
                            index=index)
    if wl.kind == "step":
        layers = shape.get("layers", wl.layers)
        return [step_layer(l, B, C, seed=s, in_dtype=wl.in_dtype, index=index)
                for l in range(layers)]
    if wl.kind == "shift":
        return shift_mix_case(B, T, C, seed=s, dtype=wl.in_dtype, prior=wl.prior, index=index)
    if wl.kind == "gate":
        return gate_case(B * T * C, seed=s, in_dtype=wl.in_dtype, out_dtype=wl.out_dtype, index=index)
    raise ValueError(wl.kind)


def shift_mix_case(B, T, C, *, seed, dtype="f16", ln=True, mixes="kvr", prior=True,
                   row_stats=True, index=5):
    """Inputs for rwkv4_shift_mix.  Draw order: x, [row offsets, row scales], x_prev,
    [ln_weight, ln_bias], mix_k, mix_v, mix_r (each mix drawn whether or not it is used, so a
    case's values do not depend on which outputs are requested)."""
    g = rng_for(index, seed)
    a = g.standard_normal((B, T, C))
    if row_stats:
        off = g.normal(0.0, 2.0, (B, T, 1))
        sc = g.uniform(0.5, 4.0, (B, T, 1))
        a = a * sc + off
    x = _as(a, dtype)
    x_prev = _normal(g, (B, C), dtype) if prior else None
    if ln:
        ln_w = g.normal(1.0, 0.25, C).astype(np.float32)
        ln_b = g.normal(0.0, 0.1, C).astype(np.float32)
    else:
        ln_w = ln_b = None
    mk = g.uniform(0.0, 1.0, C).astype(np.float32)
    mv = g.uniform(0.0, 1.0, C).astype(np.float32)
    mr = g.uniform(0.0, 1.0, C).astype(np.float32)
    return dict(B=B, T=T, C=C, x=x, x_prev=x_prev, ln_weight=ln_w, ln_bias=ln_b, ln_eps=LN_EPS,
                mix_k=mk if "k" in mixes else None, mix_v=mv if "v" in mixes else None,
                mix_r=mr if "r" in mixes else None, dtype=dtype)


def gate_case(n, *, seed, in_dtype="f16", out_dtype=None, residual=True, index=6):
    """Inputs for rwkv4_channelmix_gate over n elements.  Draw order: r, kv, [residual]."""
    g = rng_for(index, seed)
    r = _normal(g, (n,), in_dtype, sigma=2.0)
    kv = _normal(g, (n,), in_dtype)
    res = _normal(g, (n,), in_dtype) if residual else None
    return dict(n=n, r=r, kv=kv, residual=res, in_dtype=in_dtype, out_dtype=out_dtype or in_dtype)
