import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The tests load the in-tree library; build it only if nothing is built.
    lib = os.path.join(ROOT, "weight_activation_quantized_amd", "libmq.so")
    if not os.path.exists(lib):
        from weight_activation_quantized_amd import _build
        _build.build()
