import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

# The tests load the built library; build it only when nothing is built yet.
if not os.path.exists(os.path.join(ROOT, "mla_decoupled_rope_amd", "libmla.so")):
    from mla_decoupled_rope_amd import build as _build

    _build.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
