"""Host-only checks of librwkvwkv (no GPU): the library loads, exports every function
include/rwkvwkv.h declares, and rejects invalid arguments with the documented status
before anything is enqueued.  The pointers below are fake device addresses: every
call here fails validation, which runs before any HIP call, so none is dereferenced."""
import ctypes
import subprocess

import pytest

import rwkv_wkv_linear_amd as rw

L = rw.lib
P = 0x7F0000000000  # fake, 256-byte aligned device address


def p(off=0):
    return ctypes.c_void_p(P + off)


def opts(**kw):
    o = rw.Opts()
    o.size = ctypes.sizeof(rw.Opts)
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def fwd(B=2, T=8, C=16, w=p(0x10000), u=p(0x20000), k=p(0x100000), v=p(0x200000), y=p(0x300000),
        si=None, so=None, o=None):
    return L.rwkv4_wkv_forward(B, T, C, w, u, k, v, y, si, so, None,
                               ctypes.byref(o) if o is not None else None)


def test_exports_every_declared_function():
    names = rw.header_functions()
    assert set(names) >= {"rwkv4_wkv_forward", "rwkv4_wkv_step", "rwkv4_timemix_fused",
                          "rwkv_status_string", "rwkv_last_error", "rwkv4_workspace_bytes",
                          "rwkv_abi_version"}
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", rw.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in syms, f"{n} not exported by {rw.LIB_PATH}"


def test_version_and_strings():
    assert rw.rwkv_abi_version() == 1
    for code, text in [(0, "ok"), (-1, "invalid argument"), (-2, "invalid dtype"),
                       (-3, "misaligned pointer"), (-4, "HIP runtime error"),
                       (-5, "out of device memory")]:
        assert rw.status_string(code) == text
    assert rw.status_string(-99) == "unknown status"


@pytest.mark.parametrize("kw", [dict(B=0), dict(C=0), dict(T=-1), dict(B=-3)])
def test_bad_sizes(kw):
    assert fwd(**kw) == rw.RWKV_ERR_ARG
    assert "sizes" in rw.rwkv_last_error()


@pytest.mark.parametrize("name", ["w", "u", "k", "v", "y"])
def test_null_required_pointer(name):
    assert fwd(**{name: None}) == rw.RWKV_ERR_ARG


def test_null_kvy_allowed_when_T_is_zero_but_sizes_still_checked():
    # T = 0 with valid sizes would enqueue a state copy, so only the failing variant runs here
    assert fwd(T=0, B=0, k=None, v=None, y=None) == rw.RWKV_ERR_ARG


def test_too_large():
    assert fwd(B=1 << 20, T=1 << 20, C=1 << 20) == rw.RWKV_ERR_ARG


def test_bad_opts():
    o = opts(); o.size = 8
    assert fwd(o=o) == rw.RWKV_ERR_ARG and "opts->size" in rw.rwkv_last_error()
    assert fwd(o=opts(in_dtype=7)) == rw.RWKV_ERR_DTYPE
    assert fwd(o=opts(out_dtype=-1)) == rw.RWKV_ERR_DTYPE
    assert fwd(o=opts(algo=5)) == rw.RWKV_ERR_ARG
    assert fwd(o=opts(algo=4)) == rw.RWKV_ERR_ARG
    for c in (8, 48, 100, 2048, -64):
        assert fwd(o=opts(chunk_len=c)) == rw.RWKV_ERR_ARG, c
    assert fwd(o=opts(workspace=P + 4, workspace_bytes=1 << 20)) == rw.RWKV_ERR_ALIGN
    for bad in (-1, 3):
        assert fwd(o=opts(publish=bad)) == rw.RWKV_ERR_ARG and "opts->publish" in rw.rwkv_last_error()


def test_opts_without_publish_field_accepted():
    # the struct as it was before its last field: the size check passes (publish is AUTO), so
    # the call goes on to fail at the next check, the bad dtype
    o = opts(in_dtype=7)
    o.size = rw.Opts.publish.offset
    assert fwd(o=o) == rw.RWKV_ERR_DTYPE


def test_two_pass_chunk_len_limit():
    # the two-pass scan stages whole tiles in LDS (160 KB): gated 2-byte rows up to 256 tokens,
    # ungated up to 512, fp32 half of those; longer chunks (up to 1024) run only in the
    # single-launch scan, as long tiles
    for c in (512, 1024):
        o = opts(in_dtype=rw.RWKV_F16, out_dtype=rw.RWKV_F16, r=P + 0x400000, chunk_len=c,
                 algo=rw.RWKV_ALGO_TWO_PASS)
        assert fwd(T=4096, o=o) == rw.RWKV_ERR_ARG and "two-pass" in rw.rwkv_last_error()
    o = opts(in_dtype=rw.RWKV_F16, out_dtype=rw.RWKV_F16, chunk_len=1024, algo=rw.RWKV_ALGO_TWO_PASS)
    assert fwd(T=4096, o=o) == rw.RWKV_ERR_ARG and "two-pass" in rw.rwkv_last_error()
    o = opts(chunk_len=512, algo=rw.RWKV_ALGO_TWO_PASS)
    assert fwd(T=4096, o=o) == rw.RWKV_ERR_ARG and "two-pass" in rw.rwkv_last_error()
    o = opts(r=P + 0x400000, chunk_len=256, algo=rw.RWKV_ALGO_TWO_PASS)
    assert fwd(T=4096, o=o) == rw.RWKV_ERR_ARG and "two-pass" in rw.rwkv_last_error()


def test_workspace_too_small():
    o = opts(in_dtype=rw.RWKV_F16, out_dtype=rw.RWKV_F16, chunk_len=64, algo=rw.RWKV_ALGO_CHUNKED,
             workspace=P + 0x800000, workspace_bytes=16)
    assert fwd(T=4096, o=o) == rw.RWKV_ERR_ARG and "workspace" in rw.rwkv_last_error()


def test_misaligned():
    f16 = opts(in_dtype=rw.RWKV_F16, out_dtype=rw.RWKV_F16)
    assert fwd(k=p(0x100001), o=f16) == rw.RWKV_ERR_ALIGN
    assert fwd(v=p(0x200002)) == rw.RWKV_ERR_ALIGN           # fp32 needs 4-byte alignment
    assert fwd(y=p(0x300002)) == rw.RWKV_ERR_ALIGN
    assert fwd(w=p(0x10002)) == rw.RWKV_ERR_ALIGN
    assert fwd(si=p(0x500002)) == rw.RWKV_ERR_ALIGN


def test_aliasing():
    # state_out partly overlapping state_in
    assert fwd(si=p(0x500000), so=p(0x500010)) == rw.RWKV_ERR_ARG
    # y on top of k
    assert fwd(y=p(0x100000)) == rw.RWKV_ERR_ARG
    # state_out inside y
    assert fwd(so=p(0x300000)) == rw.RWKV_ERR_ARG


def test_step_validation():
    s = L.rwkv4_wkv_step
    args = [4, 16, p(0x10000), p(0x20000), p(0x100000), p(0x200000), None, p(0x300000)]
    assert s(*args, None, 1, 1, None) == rw.RWKV_ERR_ARG                    # state required
    assert s(*args, p(0x500000), 3, 1, None) == rw.RWKV_ERR_DTYPE
    assert s(*args, p(0x500000), 1, 9, None) == rw.RWKV_ERR_DTYPE
    assert s(0, 16, *args[2:], p(0x500000), 1, 1, None) == rw.RWKV_ERR_ARG   # B = 0
    a2 = list(args); a2[4] = None
    assert s(*a2, p(0x500000), 1, 1, None) == rw.RWKV_ERR_ARG                # k required


def test_timemix_validation():
    t = L.rwkv4_timemix_fused
    B, T, C = 1, 8, 16

    def call(x=p(0x100000), mix_k=p(0x30000), mix_v=p(0x40000), mix_r=p(0x50000), xk=None,
             o=None):
        return t(B, T, C, x, None, None, mix_k, mix_v, mix_r, p(0x200000), p(0x300000),
                 p(0x10000), p(0x20000), p(0x400000), xk, None, None, None, None,
                 ctypes.byref(o) if o is not None else None)

    assert call(o=opts(r=P + 0x900000)) == rw.RWKV_ERR_ARG and "opts->r" in rw.rwkv_last_error()
    assert call(mix_r=None) == rw.RWKV_ERR_ARG
    assert call(x=None) == rw.RWKV_ERR_ARG
    assert call(mix_k=None, xk=p(0x600000)) == rw.RWKV_ERR_ARG
    assert call(xk=p(0x100000)) == rw.RWKV_ERR_ARG  # xk_out on top of x


def test_last_error_is_thread_local_message():
    assert fwd(B=0) == rw.RWKV_ERR_ARG
    msg = rw.rwkv_last_error()
    assert msg and "B >= 1" in msg


def test_workspace_bytes():
    assert rw.rwkv4_workspace_bytes(1, 64, 64, 64) == 0          # one tile per chain: none needed
    assert rw.rwkv4_workspace_bytes(0, 64, 64, 0) == 0
    a = rw.rwkv4_workspace_bytes(1, 65536, 2048, 64)
    b = rw.rwkv4_workspace_bytes(1, 65536, 2048, 1024)
    assert a > b > 0
    # a 256-byte header (the error word), tiles * 4 fields * 64 channels * 8-byte
    # tagged words, and the two-pass aggregates (tiles * 64 channels * 4 fp32)
    tiles = 32 * 1024
    assert a == 256 + tiles * 4 * 64 * 8 + tiles * 64 * 16


def shift(B=2, T=8, C=16, x=p(0x100000), x_prev=None, x_last=None, ln_w=p(0x10000), ln_b=p(0x20000),
          eps=1e-5, mk=p(0x30000), mv=None, mr=p(0x50000), xk=p(0x400000), xv=None, xr=p(0x600000), dt=1):
    return L.rwkv4_shift_mix(B, T, C, x, x_prev, x_last, ln_w, ln_b, eps, mk, mv, mr, xk, xv, xr, dt, None)


def test_shift_mix_validation():
    assert shift(B=0) == rw.RWKV_ERR_ARG and "sizes" in rw.rwkv_last_error()
    assert shift(T=-1) == rw.RWKV_ERR_ARG
    assert shift(dt=5) == rw.RWKV_ERR_DTYPE
    assert shift(x=None) == rw.RWKV_ERR_ARG                          # x required when T > 0
    assert shift(ln_w=None) == rw.RWKV_ERR_ARG                       # bias without weight
    assert shift(eps=-1.0) == rw.RWKV_ERR_ARG and "ln_eps" in rw.rwkv_last_error()
    assert shift(eps=float("inf")) == rw.RWKV_ERR_ARG
    assert shift(eps=float("nan")) == rw.RWKV_ERR_ARG
    assert shift(xk=None) == rw.RWKV_ERR_ARG                         # a mix without its output
    assert shift(xv=p(0x500000)) == rw.RWKV_ERR_ARG                  # an output without its mix
    assert shift(x=p(0x100001)) == rw.RWKV_ERR_ALIGN                 # fp16 needs 2-byte alignment
    assert shift(mk=p(0x30002)) == rw.RWKV_ERR_ALIGN
    assert shift(dt=0, xr=p(0x600002)) == rw.RWKV_ERR_ALIGN          # fp32 needs 4 bytes
    assert shift(xk=p(0x100010)) == rw.RWKV_ERR_ARG                  # xk inside x
    assert shift(xr=p(0x400010)) == rw.RWKV_ERR_ARG                  # xr inside xk
    assert shift(x_last=p(0x100000)) == rw.RWKV_ERR_ARG              # x_last on top of x
    assert shift(x_prev=p(0x700000), x_last=p(0x700002)) == rw.RWKV_ERR_ARG  # partial overlap
    assert shift(x_prev=p(0x700000), xk=p(0x700000)) == rw.RWKV_ERR_ARG


def gate(n=64, r=p(0x100000), kv=p(0x200000), res=p(0x300000), y=p(0x400000), i=1, o=1):
    return L.rwkv4_channelmix_gate(n, r, kv, res, y, i, o, None)


def test_channelmix_gate_validation():
    assert gate(n=-1) == rw.RWKV_ERR_ARG
    assert gate(n=1 << 50) == rw.RWKV_ERR_ARG
    assert gate(i=4) == rw.RWKV_ERR_DTYPE and gate(o=-2) == rw.RWKV_ERR_DTYPE
    assert gate(r=None) == rw.RWKV_ERR_ARG and gate(kv=None) == rw.RWKV_ERR_ARG
    assert gate(y=None) == rw.RWKV_ERR_ARG
    assert gate(r=p(0x100001)) == rw.RWKV_ERR_ALIGN
    assert gate(i=0, res=p(0x300002)) == rw.RWKV_ERR_ALIGN
    assert gate(o=0, y=p(0x400002)) == rw.RWKV_ERR_ALIGN
    assert gate(y=p(0x100000)) == rw.RWKV_ERR_ARG                    # y on top of r
    assert gate(y=p(0x200010)) == rw.RWKV_ERR_ARG                    # y inside kv
    assert gate(y=p(0x300010)) == rw.RWKV_ERR_ARG                    # y partly over the residual
    assert gate(i=1, o=0, y=p(0x300000)) == rw.RWKV_ERR_ARG          # in place needs equal dtypes


def test_lookback_status_validation():
    flag = ctypes.c_int32(7)
    assert L.rwkv4_lookback_status(p(0), None, None) == rw.RWKV_ERR_ARG
    assert "gave_up" in rw.rwkv_last_error()
    assert L.rwkv4_lookback_status(p(4), None, ctypes.byref(flag)) == rw.RWKV_ERR_ALIGN
    assert flag.value == 0  # cleared before any check that fails


def test_chunked_workspace_size_checked_before_any_hip_call():
    # the capture query and the cached workspace come after every host-side check
    o = opts(in_dtype=rw.RWKV_F16, out_dtype=rw.RWKV_F16, algo=rw.RWKV_ALGO_TWO_PASS,
             workspace=P + 0x800000, workspace_bytes=255)
    assert fwd(T=4096, o=o) == rw.RWKV_ERR_ARG and "workspace" in rw.rwkv_last_error()


def test_noalloc_validation():
    t = L.rwkv4_timemix_fused_noalloc

    G = 1 << 30  # activations 1 GiB apart, so even the large shape below has no overlap

    def call(B=1, T=8, C=16, o=None):
        return t(B, T, C, p(1 * G), None, None, p(0x30000), p(0x40000), p(0x50000), p(2 * G), p(3 * G),
                 p(0x10000), p(0x20000), p(4 * G), None, None, None, None, None,
                 ctypes.byref(o) if o is not None else None)

    assert call(o=opts(workspace=P + 0x800000, workspace_bytes=1 << 20)) == rw.RWKV_ERR_ARG
    assert "workspace" in rw.rwkv_last_error()
    assert call(o=opts(algo=rw.RWKV_ALGO_CHUNKED)) == rw.RWKV_ERR_ARG and "CHUNKED" in rw.rwkv_last_error()
    # 512 channel tiles x 33 time tiles of 128 tokens: more aggregates than the 16 MiB scratch holds
    big = opts(in_dtype=rw.RWKV_F16, out_dtype=rw.RWKV_F16)
    assert call(T=4160, C=32768, o=big) == rw.RWKV_ERR_ARG and "scratch" in rw.rwkv_last_error()
    assert call(B=0) == rw.RWKV_ERR_ARG
