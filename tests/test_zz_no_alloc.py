"""rwkv4_timemix_fused_noalloc (no device allocation; the library's static scratch) against the
existing entry point rwkv4_timemix_fused, called through the C ABI: two calls in a row, the
second on a smaller input (the scratch keeps the first call's aggregates), each compared with
the allocating entry point on the same inputs and with the fp64 oracle at the fp16 bar, and
bit for bit with the allocating entry point's two-pass scan (the same kernels)."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import TOL, check_output, check_state, host, note, to_dev, torch


def _call(entry, case, algo, workspace=None):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    B, T, C = case["B"], case["T"], case["C"]
    d = {n: to_dev(case[n]) for n in ("x", "x_prev", "mix_k", "mix_v", "mix_r", "k", "v", "w", "u", "state_in")}
    y = t.full((B, T, C), float("nan"), dtype=t.float16, device="cuda:0")
    so = t.full((3, B, C), float("nan"), device="cuda:0")
    xl = t.full((B, C), float("nan"), dtype=t.float16, device="cuda:0")
    o = rw.Opts()
    o.size = ctypes.sizeof(rw.Opts)
    o.in_dtype = o.out_dtype = rw.RWKV_F16
    o.algo = {"auto": rw.RWKV_ALGO_AUTO, "two_pass": rw.RWKV_ALGO_TWO_PASS}[algo]
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel()
    vp = lambda tt: ctypes.c_void_p(tt.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(t.cuda.current_stream().cuda_stream)
    st = getattr(rw.lib, entry)(B, T, C, vp(d["x"]), vp(d["x_prev"]), vp(xl), vp(d["mix_k"]), vp(d["mix_v"]),
                                vp(d["mix_r"]), vp(d["k"]), vp(d["v"]), vp(d["w"]), vp(d["u"]), vp(y), None, None,
                                vp(d["state_in"]), vp(so), stream, ctypes.byref(o))
    assert st == rw.RWKV_OK, rw.rwkv_last_error()
    t.cuda.synchronize()
    return y, so, xl


def test_noalloc_matches_the_allocating_entry_point():
    import rwkv_wkv_linear_amd as rw
    t = torch()
    cases = [wi.timemix_case(1, 1024, 5120, seed=131, prior=True),   # the 14B layer shape, 640 tiles
             wi.timemix_case(2, 300, 256, seed=132, prior=True)]     # then a smaller call
    for case in cases:
        B, T, C = case["B"], case["T"], case["C"]
        ref = oracle.timemix(case)
        note(f"noalloc timemix B={B} T={T} C={C}")
        y0, s0, x0 = _call("rwkv4_timemix_fused_noalloc", case, "auto")
        note(f"allocating timemix B={B} T={T} C={C} (auto and two-pass)")
        ya, sa, xa = _call("rwkv4_timemix_fused", case, "auto")
        ws = t.zeros(rw.rwkv4_workspace_bytes(B, T, C, 0), dtype=t.uint8, device="cuda:0")
        y2, s2, x2 = _call("rwkv4_timemix_fused", case, "two_pass", ws)
        what = f"noalloc B{B} T{T} C{C}"
        # the same kernels as the allocating two-pass scan: bit for bit
        assert t.equal(y0, y2) and t.equal(s0, s2) and t.equal(x0, x2), f"{what}: differs from the two-pass call"
        # and the allocating entry point's default (single-pass) result to the parity bar
        d = np.max(np.abs(host(y0) - host(ya)) / np.maximum(ref["scale"], 2.0 ** -14))
        note(f"{what}: vs the allocating entry point's auto call: {d:.3e}")
        assert d <= TOL["f16"], f"{what}: {d:.3e} from the allocating entry point"
        assert t.equal(x0, xa)
        check_output(host(y0), ref, TOL["f16"], what, out_dtype="f16")
        check_state(host(s0), ref, what)
        assert np.array_equal(host(x0), ref["x_last"])
