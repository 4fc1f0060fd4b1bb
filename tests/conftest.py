import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

# The tests load the built library: rebuild it when it is missing or was built
# from other sources than the ones in the tree (a hash of every HIP source and
# header, recorded next to the library by the build).
import importlib.util  # noqa: E402

_spec = importlib.util.spec_from_file_location("_mla_build", os.path.join(ROOT, "mla_decoupled_rope_amd", "build.py"))
_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_build)
if not _build.is_current():
    print("libmla.so is missing or older than its sources: building it", flush=True)
    _build.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
