"""Build librwkvwkv.so (gfx950 only) in-tree with hipcc.

    python -m rwkv_wkv_linear_amd.build [--verbose]

The library is written next to this file; the Python binding loads it from there.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librwkvwkv.so")
# the benchmark's bandwidth ceilings (stream_ceiling.hip): a library of its own, not linked into
# librwkvwkv and not part of its ABI
CEIL_LIB = os.path.join(HERE, "libwkvceiling.so")
# (source, extra flags, object name): wkv_kernels.hip is compiled once per input dtype
# (-DRWKV_TU_IN = rwkv_dtype code), so its many kernel instantiations build in parallel
SOURCES = [("wkv_kernels.hip", ["-DRWKV_TU_IN=0"], "wkv_kernels_f32"),
           ("wkv_kernels.hip", ["-DRWKV_TU_IN=1"], "wkv_kernels_f16"),
           ("wkv_kernels.hip", ["-DRWKV_TU_IN=2"], "wkv_kernels_bf16"),
           ("mix_kernels.hip", [], "mix_kernels"),
           ("rwkvwkv_abi.hip", [], "rwkvwkv_abi")]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    # no packed FP32 instructions anywhere (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmds, verbose):
    """Run the commands in parallel; raise with their diagnostics if any fails."""
    # hipcc's host pass does not know the packed-fp32 feature name; drop that warning only
    noise = "'-packed-fp32-ops' is not a recognized feature"
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    failed = []
    for cmd, p in zip(cmds, procs):
        _, err = p.communicate()
        errlines = [l for l in err.splitlines() if noise not in l]
        if p.returncode != 0:
            failed.append(" ".join(cmd[-3:]) + "\n" + "\n".join(errlines))
        elif verbose and errlines:
            print("\n".join(errlines), file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(failed))


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source to an object in parallel, then link the shared library."""
    tag = "%d" % os.getpid()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(objdir, "%s.%s.o" % (name, tag)) for _, _, name in SOURCES]
    _run([[hipcc(), *HIPCC_FLAGS, *flags, *(extra_flags or []), *inc, "-c", os.path.join(CSRC, src), "-o", o]
          for (src, flags, _), o in zip(SOURCES, objs)], verbose)
    tmp = LIB + ".tmp" + tag
    ctmp = CEIL_LIB + ".tmp" + tag
    try:
        _run([[hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp],
              [hipcc(), *HIPCC_FLAGS, "-shared", os.path.join(CSRC, "stream_ceiling.hip"), "-o", ctmp]], verbose)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    os.replace(tmp, LIB)
    os.replace(ctmp, CEIL_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
    print(LIB)
