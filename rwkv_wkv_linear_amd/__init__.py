"""Python binding of librwkvwkv: the RWKV-4 WKV time-mixing path on AMD MI355X (gfx950).

Thin ctypes marshalling over the C ABI in include/rwkvwkv.h -- every step of the
computation runs in the library's HIP kernels.  Functions carry the C names and
take torch tensors (device memory and streams only); they check shapes, dtypes,
devices and contiguity, pass data pointers and the current HIP stream, and raise
RwkvError on a non-OK status.  The library loads on first use and raises
ImportError if it is not built (``python -m rwkv_wkv_linear_amd.build``); there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librwkvwkv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "rwkvwkv.h")

RWKV_OK, RWKV_ERR_ARG, RWKV_ERR_DTYPE, RWKV_ERR_ALIGN, RWKV_ERR_HIP, RWKV_ERR_NOMEM = 0, -1, -2, -3, -4, -5
RWKV_F32, RWKV_F16, RWKV_BF16 = 0, 1, 2
RWKV_ALGO_AUTO, RWKV_ALGO_SEQUENTIAL, RWKV_ALGO_CHUNKED, RWKV_ALGO_TWO_PASS = 0, 1, 2, 3
_ALGOS = {"auto": 0, "sequential": 1, "chunked": 2, "two_pass": 3, 0: 0, 1: 1, 2: 2, 3: 3}
RWKV_PUBLISH_AUTO, RWKV_PUBLISH_L2_FIRST, RWKV_PUBLISH_WRITE_THROUGH = 0, 1, 2
_PUBLISH = {"auto": 0, "l2_first": 1, "write_through": 2, 0: 0, 1: 1, 2: 2}


class Opts(ctypes.Structure):
    """Mirror of struct rwkv4_opts."""
    _fields_ = [
        ("size", ctypes.c_uint32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("r", ctypes.c_void_p),
        ("chunk_len", ctypes.c_int32),
        ("algo", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("publish", ctypes.c_int32),
    ]


class RwkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"librwkvwkv status {status} ({status_string(status)}): {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run: python -m rwkv_wkv_linear_amd.build")
    # torch ships its own HIP runtime (SONAME libamdhip64.so.7, loaded by its unversioned
    # file name).  Loading torch first makes the library's libamdhip64.so.7 dependency
    # resolve to that same runtime; loading the library first would leave two HIP runtimes
    # in the process, and the second one to initialise finds no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, fp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.rwkv4_wkv_forward.argtypes = [i64, i64, i64, fp, fp, vp, vp, vp, fp, fp, vp, ctypes.POINTER(Opts)]
    lib.rwkv4_wkv_forward.restype = ctypes.c_int
    lib.rwkv4_wkv_step.argtypes = [i64, i64, fp, fp, vp, vp, vp, vp, fp, ctypes.c_int, ctypes.c_int, vp]
    lib.rwkv4_wkv_step.restype = ctypes.c_int
    lib.rwkv4_timemix_fused.argtypes = [i64, i64, i64, vp, vp, vp, fp, fp, fp, vp, vp, fp, fp, vp, vp, vp,
                                        fp, fp, vp, ctypes.POINTER(Opts)]
    lib.rwkv4_timemix_fused.restype = ctypes.c_int
    lib.rwkv4_timemix_fused_noalloc.argtypes = lib.rwkv4_timemix_fused.argtypes
    lib.rwkv4_timemix_fused_noalloc.restype = ctypes.c_int
    lib.rwkv4_shift_mix.argtypes = [i64, i64, i64, vp, vp, vp, fp, fp, ctypes.c_float, fp, fp, fp, vp, vp, vp,
                                    ctypes.c_int, vp]
    lib.rwkv4_shift_mix.restype = ctypes.c_int
    lib.rwkv4_channelmix_gate.argtypes = [i64, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp]
    lib.rwkv4_channelmix_gate.restype = ctypes.c_int
    lib.rwkv_status_string.argtypes = [ctypes.c_int]
    lib.rwkv_status_string.restype = ctypes.c_char_p
    lib.rwkv_last_error.argtypes = []
    lib.rwkv_last_error.restype = ctypes.c_char_p
    lib.rwkv4_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int32]
    lib.rwkv4_workspace_bytes.restype = ctypes.c_size_t
    lib.rwkv4_lookback_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32)]
    lib.rwkv4_lookback_status.restype = ctypes.c_int
    lib.rwkv_abi_version.argtypes = []
    lib.rwkv_abi_version.restype = ctypes.c_int
    return lib


_lib = None


def _get_lib():
    """The loaded library (loaded on first use; raises ImportError if it is not built)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def __getattr__(name):
    # `rwkv_wkv_linear_amd.lib` loads the library on first access; importing the package
    # alone does not, so the build step can import it while no library exists yet
    if name == "lib":
        return _get_lib()
    raise AttributeError(name)


def header_functions(path: str = HEADER_PATH):
    """Names of the functions include/rwkvwkv.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(rwkv[0-9a-z_]*)\s*\(", text)


def status_string(status: int) -> str:
    return _get_lib().rwkv_status_string(int(status)).decode()


def rwkv_status_string(status: int) -> str:
    return status_string(status)


def rwkv_last_error() -> str:
    return _get_lib().rwkv_last_error().decode()


def rwkv_abi_version() -> int:
    return _get_lib().rwkv_abi_version()


def rwkv4_workspace_bytes(B: int, T: int, C: int, chunk_len: int = 0) -> int:
    return int(_get_lib().rwkv4_workspace_bytes(B, T, C, chunk_len))


# ----------------------------------------------------------------------------- tensor marshalling

def _torch():
    import torch
    return torch


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float32:
        return RWKV_F32
    if dt == torch.float16:
        return RWKV_F16
    if dt == torch.bfloat16:
        return RWKV_BF16
    raise TypeError(f"unsupported dtype {dt}: float32, float16 or bfloat16")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, shape=None, dtype=None, device=None):
    if t is None:
        return
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _check(status):
    if status != RWKV_OK:
        raise RwkvError(status, rwkv_last_error())


def _opts(in_dtype, out_dtype, r=None, chunk_len=0, algo="auto", workspace=None, publish="auto"):
    o = Opts()
    o.size = ctypes.sizeof(Opts)
    o.in_dtype = in_dtype
    o.out_dtype = out_dtype
    o.r = _ptr(r)
    o.chunk_len = int(chunk_len)
    o.algo = _ALGOS[algo]
    o.publish = _PUBLISH[publish]
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    return o


def rwkv4_wkv_forward(k, v, w, u, y=None, state_in=None, state_out=None, *, r=None, out_dtype=None,
                      chunk_len=0, algo="auto", workspace=None, publish="auto", stream=None):
    """y = WKV(k, v) (or sigmoid(r) * WKV when r is given); fills state_out if given.
    k, v, r: [B, T, C] float32/float16/bfloat16; w, u: [C] float32; states: [3, B, C] float32."""
    torch = _torch()
    B, T, C = k.shape
    dev = k.device
    _need(k, "k", dtype=k.dtype)
    _need(v, "v", (B, T, C), k.dtype, dev)
    _need(r, "r", (B, T, C), k.dtype, dev)
    _need(w, "w", (C,), torch.float32, dev)
    _need(u, "u", (C,), torch.float32, dev)
    _need(state_in, "state_in", (3, B, C), torch.float32, dev)
    _need(state_out, "state_out", (3, B, C), torch.float32, dev)
    odt = out_dtype or (y.dtype if y is not None else k.dtype)
    if y is None:
        y = torch.empty((B, T, C), dtype=odt, device=dev)
    _need(y, "y", (B, T, C), odt, dev)
    _need(workspace, "workspace", device=dev)
    o = _opts(_dtype_code(k.dtype), _dtype_code(odt), r, chunk_len, algo, workspace, publish)
    with torch.cuda.device(dev):
        _check(_get_lib().rwkv4_wkv_forward(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                     _ptr(state_in), _ptr(state_out), _stream(stream, dev),
                                     ctypes.byref(o)))
    return y


def rwkv4_wkv_step(k, v, r, w, u, state, y=None, *, out_dtype=None, stream=None):
    """One decode token: k, v, r [B, C] (r may be None); state [3, B, C] updated in place."""
    torch = _torch()
    B, C = k.shape
    dev = k.device
    _need(k, "k", dtype=k.dtype)
    _need(v, "v", (B, C), k.dtype, dev)
    _need(r, "r", (B, C), k.dtype, dev)
    _need(w, "w", (C,), torch.float32, dev)
    _need(u, "u", (C,), torch.float32, dev)
    _need(state, "state", (3, B, C), torch.float32, dev)
    odt = out_dtype or (y.dtype if y is not None else k.dtype)
    if y is None:
        y = torch.empty((B, C), dtype=odt, device=dev)
    _need(y, "y", (B, C), odt, dev)
    with torch.cuda.device(dev):
        _check(_get_lib().rwkv4_wkv_step(B, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r), _ptr(y),
                                  _ptr(state), _dtype_code(k.dtype), _dtype_code(odt),
                                  _stream(stream, dev)))
    return y


def rwkv4_timemix_fused(x, x_prev, mix_k, mix_v, mix_r, k, v, w, u, y=None, *, xk_out=None,
                        xv_out=None, x_last=None, state_in=None, state_out=None, out_dtype=None,
                        chunk_len=0, algo="auto", workspace=None, publish="auto", stream=None,
                        _entry="rwkv4_timemix_fused"):
    """Token shift + WKV + receptance gate: y = sigmoid(xr) * WKV(k, v).
    x, k, v [B, T, C]; x_prev, x_last [B, C] (x's dtype); mix_* [C] float32."""
    torch = _torch()
    B, T, C = x.shape
    dev = x.device
    dt = x.dtype
    _need(x, "x", dtype=dt)
    _need(x_prev, "x_prev", (B, C), dt, dev)
    _need(x_last, "x_last", (B, C), dt, dev)
    for name, m in (("mix_k", mix_k), ("mix_v", mix_v), ("mix_r", mix_r), ("w", w), ("u", u)):
        _need(m, name, (C,), torch.float32, dev)
    _need(k, "k", (B, T, C), dt, dev)
    _need(v, "v", (B, T, C), dt, dev)
    _need(xk_out, "xk_out", (B, T, C), dt, dev)
    _need(xv_out, "xv_out", (B, T, C), dt, dev)
    _need(state_in, "state_in", (3, B, C), torch.float32, dev)
    _need(state_out, "state_out", (3, B, C), torch.float32, dev)
    odt = out_dtype or (y.dtype if y is not None else dt)
    if y is None:
        y = torch.empty((B, T, C), dtype=odt, device=dev)
    _need(y, "y", (B, T, C), odt, dev)
    _need(workspace, "workspace", device=dev)
    o = _opts(_dtype_code(dt), _dtype_code(odt), None, chunk_len, algo, workspace, publish)
    with torch.cuda.device(dev):
        _check(getattr(_get_lib(), _entry)(B, T, C, _ptr(x), _ptr(x_prev), _ptr(x_last), _ptr(mix_k),
                                       _ptr(mix_v), _ptr(mix_r), _ptr(k), _ptr(v), _ptr(w), _ptr(u),
                                       _ptr(y), _ptr(xk_out), _ptr(xv_out), _ptr(state_in),
                                       _ptr(state_out), _stream(stream, dev), ctypes.byref(o)))
    return y


def rwkv4_timemix_fused_noalloc(x, x_prev, mix_k, mix_v, mix_r, k, v, w, u, y=None, **kw):
    """rwkv4_timemix_fused on the library's static scratch (no device allocation; no workspace
    argument; the sequential kernel or the two-pass scan).  The caller passes y (and every other
    output it wants) when it cannot allocate either."""
    if kw.get("workspace") is not None:
        raise ValueError("rwkv4_timemix_fused_noalloc takes no workspace")
    return rwkv4_timemix_fused(x, x_prev, mix_k, mix_v, mix_r, k, v, w, u, y, _entry="rwkv4_timemix_fused_noalloc",
                               **kw)


def rwkv4_lookback_status(workspace=None, *, stream=None, device=None):
    """True when a look-back wait of a single-launch chunked scan on `workspace` (a tensor passed
    as the calls' workspace; None: the library-cached workspace of `stream`, by default the
    current stream of `device`) gave up since it was last checked; clears the flag.  Waits for
    the stream's work first."""
    torch = _torch()
    dev = workspace.device if workspace is not None else (device or torch.device("cuda", torch.cuda.current_device()))
    _need(workspace, "workspace", device=dev)
    flag = ctypes.c_int32(0)
    with torch.cuda.device(dev):
        _check(_get_lib().rwkv4_lookback_status(_ptr(workspace), _stream(stream, dev), ctypes.byref(flag)))
    return bool(flag.value)


def rwkv4_shift_mix(x, x_prev=None, *, ln_weight=None, ln_bias=None, ln_eps=1e-5, mix_k=None, mix_v=None,
                    mix_r=None, xk=None, xv=None, xr=None, x_last=None, stream=None):
    """Pre-LN token-shift prologue: n = LayerNorm(x) over the channels (x itself when ln_weight
    is None); for each given mix, out = mix * n_t + (1 - mix) * n_{t-1} with n_{-1} = x_prev.
    x [B, T, C]; x_prev, x_last [B, C] (x's dtype; x_last may be x_prev itself); ln_*, mix_* [C]
    float32.  Outputs not passed are allocated for each given mix.  Returns (xk, xv, xr, x_last)
    (None where not requested)."""
    torch = _torch()
    B, T, C = x.shape
    dev, dt = x.device, x.dtype
    _need(x, "x", dtype=dt)
    _need(x_prev, "x_prev", (B, C), dt, dev)
    _need(x_last, "x_last", (B, C), dt, dev)
    for name, m in (("ln_weight", ln_weight), ("ln_bias", ln_bias), ("mix_k", mix_k), ("mix_v", mix_v),
                    ("mix_r", mix_r)):
        _need(m, name, (C,), torch.float32, dev)
    outs = []
    for name, mix, o in (("xk", mix_k, xk), ("xv", mix_v, xv), ("xr", mix_r, xr)):
        if mix is not None and o is None:
            o = torch.empty((B, T, C), dtype=dt, device=dev)
        _need(o, name, (B, T, C), dt, dev)
        outs.append(o)
    with torch.cuda.device(dev):
        _check(_get_lib().rwkv4_shift_mix(B, T, C, _ptr(x), _ptr(x_prev), _ptr(x_last), _ptr(ln_weight),
                                          _ptr(ln_bias), float(ln_eps), _ptr(mix_k), _ptr(mix_v), _ptr(mix_r),
                                          _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _dtype_code(dt),
                                          _stream(stream, dev)))
    return outs[0], outs[1], outs[2], x_last


def rwkv4_channelmix_gate(r, kv, residual=None, y=None, *, out_dtype=None, stream=None):
    """y = residual + kv / (1 + e^{-r}) elementwise (residual None: 0).  r, kv, residual share a
    shape and dtype; y (allocated if None) has that shape and out_dtype (default r's dtype) and
    may be residual itself."""
    torch = _torch()
    dev, dt = r.device, r.dtype
    _need(r, "r", dtype=dt)
    _need(kv, "kv", tuple(r.shape), dt, dev)
    _need(residual, "residual", tuple(r.shape), dt, dev)
    odt = out_dtype or (y.dtype if y is not None else dt)
    if y is None:
        y = torch.empty(r.shape, dtype=odt, device=dev)
    _need(y, "y", tuple(r.shape), odt, dev)
    with torch.cuda.device(dev):
        _check(_get_lib().rwkv4_channelmix_gate(r.numel(), _ptr(r), _ptr(kv), _ptr(residual), _ptr(y),
                                                _dtype_code(dt), _dtype_code(odt), _stream(stream, dev)))
    return y


__all__ = [
    "lib", "LIB_PATH", "Opts", "RwkvError", "header_functions", "status_string",
    "rwkv4_wkv_forward", "rwkv4_wkv_step", "rwkv4_timemix_fused", "rwkv_status_string",
    "rwkv_last_error", "rwkv4_workspace_bytes", "rwkv_abi_version", "rwkv4_shift_mix",
    "rwkv4_channelmix_gate", "rwkv4_lookback_status", "rwkv4_timemix_fused_noalloc",
]
