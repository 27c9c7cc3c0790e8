"""A look-back that gives up is visible to the caller: rwkv4_lookback_status reports it and clears
it.  The failure is forced from the host, the way the header documents: a nonzero error word
(the first 4 bytes of a caller workspace) makes every look-back on the workspace give up at
once, so every kernel still exits normally.  Tiles of the first time tile wait for nothing and
stay correct; every later tile's outputs are NaN.  After the status call clears the word, the
same call is correct again."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
import wkv_inputs as wi
from gpu_util import TOL, check_output, check_state, host, note, to_dev, torch


@pytest.mark.parametrize("chunk", [16, 64, 128, 256])
def test_forced_give_up_is_reported_and_cleared(chunk):
    import rwkv_wkv_linear_amd as rw
    t = torch()
    B, T, C = 2, 1000, 192
    case = wi.forward_case(B, T, C, seed=101, in_dtype="f16", gated=True, prior=True)
    ref = oracle.forward(case)
    d = {n: to_dev(case[n]) for n in ("k", "v", "r", "w", "u", "state_in")}
    ws = t.zeros(rw.rwkv4_workspace_bytes(B, T, C, chunk), dtype=t.uint8, device="cuda:0")

    def call():
        y = t.full((B, T, C), float("nan"), dtype=t.float16, device="cuda:0")
        so = t.full((3, B, C), float("nan"), device="cuda:0")
        rw.rwkv4_wkv_forward(d["k"], d["v"], d["w"], d["u"], y=y, state_in=d["state_in"], state_out=so,
                             r=d["r"], algo="chunked", chunk_len=chunk, workspace=ws)
        return y, so

    note(f"lookback status on a clean workspace chunk={chunk}")
    y, so = call()
    assert rw.rwkv4_lookback_status(ws) is False
    check_output(host(y), ref, TOL["f16"], f"clean workspace chunk={chunk}", out_dtype="f16")

    ws.view(t.int32)[0] = 1  # the error word: every look-back on the workspace gives up at once
    t.cuda.synchronize()
    note(f"forced give-up chunk={chunk}")
    y, so = call()
    t.cuda.synchronize()
    yh = host(y)
    assert np.all(np.isnan(yh[:, chunk:])), "a tile that waited produced numbers"
    assert np.all(np.isnan(host(so)[:2])), "the final state came from a tile that waited"
    first = dict(ref, y=ref["y"][:, :chunk], scale=ref["scale"][:, :chunk])
    check_output(yh[:, :chunk], first, TOL["f16"], f"first time tile under a forced give-up chunk={chunk}",
                 out_dtype="f16")
    assert rw.rwkv4_lookback_status(ws) is True
    assert rw.rwkv4_lookback_status(ws) is False, "the status call did not clear the error word"

    note(f"after clearing chunk={chunk}")
    y, so = call()
    assert rw.rwkv4_lookback_status(ws) is False
    check_output(host(y), ref, TOL["f16"], f"after clearing chunk={chunk}", out_dtype="f16")
    check_state(host(so), ref, f"after clearing chunk={chunk}")


def test_status_of_the_cached_workspace():
    """With no workspace argument the status reads the library-cached workspace of the stream:
    clear after normal calls, and clear on a stream that never ran a chunked scan."""
    import rwkv_wkv_linear_amd as rw
    t = torch()
    case = wi.forward_case(1, 700, 128, seed=102, in_dtype="f16", out_dtype="f32")
    ref = oracle.forward(case)
    d = {n: to_dev(case[n]) for n in ("k", "v", "w", "u")}
    note("lookback status, cached workspace")
    y = rw.rwkv4_wkv_forward(d["k"], d["v"], d["w"], d["u"], out_dtype=t.float32, algo="chunked")
    assert rw.rwkv4_lookback_status() is False
    check_output(host(y), ref, TOL["f16"], "cached workspace")
    assert rw.rwkv4_lookback_status(stream=t.cuda.Stream()) is False
