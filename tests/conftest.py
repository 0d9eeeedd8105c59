import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # Build the HIP library only when nothing is built yet (a fresh checkout);
    # an existing build is used as it is.
    lib = os.path.join(ROOT, "tensor_linear_amd", "libtplinear.so")
    if not os.path.exists(lib):
        from tensor_linear_amd import build as _b
        _b.build()
