import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def _ensure_built():
    """Build what is missing (the library and the oracle travel prebuilt in normal use)."""
    lib = os.path.join(ROOT, "rwkv_wkv_linear_amd", "librwkvwkv.so")
    if not os.path.exists(lib):
        from rwkv_wkv_linear_amd.build import build
        build()
    import oracle
    oracle.build(force=False)


_ensure_built()
