"""The entry points inside a captured HIP graph: 40 decode layers (rwkv4_wkv_step) and a
two-pass prefill (rwkv4_wkv_forward with RWKV_ALGO_TWO_PASS and an explicit workspace) are
captured once and replayed several times, with the program's own eager work and
synchronisations between replays; every replay must equal eager launches of the same calls
bit for bit, and the decode replay is checked against the fp64 oracle as well."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import TOL, check_output, check_state, host, note, to_dev, torch

LAYERS, B, C = 40, 32, 1024


def _layers():
    return [wi.step_layer(l, B, C, seed=77) for l in range(LAYERS)]


def test_decode_40_layers_graph_replays_equal_eager():
    import rwkv_wkv_linear_amd as rw
    t = torch()
    layers = _layers()
    dev_layers = [{n: to_dev(layer[n]) for n in ("k", "v", "r", "w", "u", "state")} for layer in layers]

    # eager reference: 40 separate step calls
    eager_state = [d["state"].clone() for d in dev_layers]
    eager_y = [t.empty((B, C), dtype=t.float16, device="cuda:0") for _ in range(LAYERS)]
    note(f"decode {LAYERS} layers eager B={B} C={C}")
    for d, st, y in zip(dev_layers, eager_state, eager_y):
        rw.rwkv4_wkv_step(d["k"], d["v"], d["r"], d["w"], d["u"], st, y=y)
    t.cuda.synchronize()

    # the same 40 calls captured into one graph over static buffers
    g_state = [d["state"].clone() for d in dev_layers]
    g_y = [t.empty((B, C), dtype=t.float16, device="cuda:0") for _ in range(LAYERS)]
    graph = t.cuda.CUDAGraph()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    note("decode graph capture")
    with t.cuda.stream(side):
        with t.cuda.graph(graph):
            for d, st, y in zip(dev_layers, g_state, g_y):
                rw.rwkv4_wkv_step(d["k"], d["v"], d["r"], d["w"], d["u"], st, y=y)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    for rep in range(3):
        for st, d in zip(g_state, dev_layers):   # eager reset between replays
            st.copy_(d["state"])
        for y in g_y:
            y.fill_(float("nan"))
        t.cuda.synchronize()
        note(f"decode graph replay {rep}")
        graph.replay()
        t.cuda.synchronize()
        for l in range(LAYERS):
            assert t.equal(g_y[l], eager_y[l]), f"replay {rep} layer {l}: y differs from eager"
            assert t.equal(g_state[l], eager_state[l]), f"replay {rep} layer {l}: state differs from eager"
    for l in (0, LAYERS - 1):
        ref = oracle.step(layers[l])
        check_output(host(g_y[l]), ref, TOL["f16"], f"graph decode layer {l}", out_dtype="f16")
        check_state(host(g_state[l]), ref, f"graph decode layer {l}")


@pytest.mark.parametrize("chunk", [64, 128])
def test_two_pass_forward_graph_replays_equal_eager(chunk):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    Bf, T, Cf = 2, 1500, 320
    cases = [wi.forward_case(Bf, T, Cf, seed=90 + i, in_dtype="f16", gated=True, prior=True) for i in range(3)]
    ws = t.zeros(rw.rwkv4_workspace_bytes(Bf, T, Cf, chunk), dtype=t.uint8, device="cuda:0")
    names = ("k", "v", "r", "state_in")
    static = {n: to_dev(cases[0][n]) for n in names}
    w, u = to_dev(cases[0]["w"]), to_dev(cases[0]["u"])
    y = t.empty((Bf, T, Cf), dtype=t.float16, device="cuda:0")
    so = t.empty((3, Bf, Cf), device="cuda:0")

    def call(src, yy, ss):
        rw.rwkv4_wkv_forward(src["k"], src["v"], w, u, y=yy, state_in=src["state_in"], state_out=ss,
                             r=src["r"], algo="two_pass", chunk_len=chunk, workspace=ws)

    graph = t.cuda.CUDAGraph()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    note(f"two-pass forward graph capture chunk={chunk}")
    with t.cuda.stream(side):
        with t.cuda.graph(graph):
            call(static, y, so)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    for rep, case in enumerate(cases):
        src = {n: to_dev(case[n]) for n in names}
        ye = t.empty_like(y)
        se = t.empty_like(so)
        note(f"two-pass forward eager {rep} chunk={chunk}")
        call(src, ye, se)
        for n in names:                      # new inputs into the graph's static buffers
            static[n].copy_(src[n])
        y.fill_(float("nan"))
        t.cuda.synchronize()
        note(f"two-pass forward graph replay {rep} chunk={chunk}")
        graph.replay()
        t.cuda.synchronize()
        assert t.equal(y, ye) and t.equal(so, se), f"replay {rep}: differs from eager"
        ref = oracle.forward(case)
        check_output(host(y), ref, TOL["f16"], f"graph two-pass replay {rep}", out_dtype="f16")
        check_state(host(so), ref, f"graph two-pass replay {rep}")


def test_auto_forward_under_capture_takes_two_pass():
    """AUTO on a capturing stream takes the two-pass scan (no per-launch epoch), so replays with
    new inputs in the graph's buffers give the right answers; each replay equals an eager
    two-pass call bit for bit and the oracle within the bar."""
    import rwkv_wkv_linear_amd as rw
    t = torch()
    Bf, T, Cf = 1, 1100, 512
    cases = [wi.forward_case(Bf, T, Cf, seed=110 + i, in_dtype="f16", gated=True, prior=True) for i in range(3)]
    ws = t.zeros(rw.rwkv4_workspace_bytes(Bf, T, Cf, 0), dtype=t.uint8, device="cuda:0")
    names = ("k", "v", "r", "state_in")
    static = {n: to_dev(cases[0][n]) for n in names}
    w, u = to_dev(cases[0]["w"]), to_dev(cases[0]["u"])
    y = t.empty((Bf, T, Cf), dtype=t.float16, device="cuda:0")
    so = t.empty((3, Bf, Cf), device="cuda:0")
    graph = t.cuda.CUDAGraph()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    note("auto forward graph capture")
    with t.cuda.stream(side):
        with t.cuda.graph(graph):
            rw.rwkv4_wkv_forward(static["k"], static["v"], w, u, y=y, state_in=static["state_in"], state_out=so,
                                 r=static["r"], workspace=ws)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    for rep, case in enumerate(cases):
        src = {n: to_dev(case[n]) for n in names}
        ye, se = t.empty_like(y), t.empty_like(so)
        note(f"two-pass eager {rep}")
        rw.rwkv4_wkv_forward(src["k"], src["v"], w, u, y=ye, state_in=src["state_in"], state_out=se, r=src["r"],
                             algo="two_pass", workspace=ws)
        for n in names:
            static[n].copy_(src[n])
        y.fill_(float("nan"))
        t.cuda.synchronize()
        note(f"auto forward graph replay {rep}")
        graph.replay()
        t.cuda.synchronize()
        assert t.equal(y, ye) and t.equal(so, se), f"replay {rep}: differs from the eager two-pass call"
        ref = oracle.forward(case)
        check_output(host(y), ref, TOL["f16"], f"graph auto replay {rep}", out_dtype="f16")
        check_state(host(so), ref, f"graph auto replay {rep}")


def test_capture_refuses_what_cannot_replay():
    """On a capturing stream the single-launch chunked scan (explicit, or a chunk_len above the
    longest tile staged in LDS, 256 tokens for gated 2-byte rows, which only it runs) and the
    library-cached workspace are refused before anything is enqueued; a call whose T fits in one
    tile needs neither and is captured as it is."""
    import rwkv_wkv_linear_amd as rw
    t = torch()
    B1, T1, C1 = 1, 600, 128
    case = wi.forward_case(B1, T1, C1, seed=120, in_dtype="f16", gated=True, prior=True)
    d = {n: to_dev(case[n]) for n in ("k", "v", "r", "w", "u", "state_in")}
    ws = t.zeros(rw.rwkv4_workspace_bytes(B1, T1, C1, 0), dtype=t.uint8, device="cuda:0")
    short = wi.forward_case(1, 100, C1, seed=121, in_dtype="f16", gated=True, prior=True)
    ds = {n: to_dev(short[n]) for n in ("k", "v", "r", "w", "u", "state_in")}
    y = t.empty((B1, T1, C1), dtype=t.float16, device="cuda:0")
    ys = t.empty((1, 100, C1), dtype=t.float16, device="cuda:0")
    graph = t.cuda.CUDAGraph()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    refused = []
    note("capture refusals")
    with t.cuda.stream(side):
        with t.cuda.graph(graph):
            for kw in (dict(algo="chunked", workspace=ws), dict(algo="auto"), dict(algo="two_pass"),
                       dict(algo="auto", chunk_len=512, workspace=ws)):
                try:
                    rw.rwkv4_wkv_forward(d["k"], d["v"], d["w"], d["u"], y=y, state_in=d["state_in"], r=d["r"], **kw)
                except rw.RwkvError as e:
                    refused.append((kw.get("algo"), e.status))
            rw.rwkv4_wkv_forward(ds["k"], ds["v"], ds["w"], ds["u"], y=ys, state_in=ds["state_in"], r=ds["r"],
                                 chunk_len=128)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    assert refused == [("chunked", rw.RWKV_ERR_ARG), ("auto", rw.RWKV_ERR_ARG), ("two_pass", rw.RWKV_ERR_ARG),
                       ("auto", rw.RWKV_ERR_ARG)], refused
    ys.fill_(float("nan"))
    t.cuda.synchronize()
    graph.replay()
    t.cuda.synchronize()
    check_output(host(ys), oracle.forward(short), TOL["f16"], "captured one-tile call", out_dtype="f16")
