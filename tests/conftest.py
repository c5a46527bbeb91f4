import os
import shutil
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

LIB = os.path.join(ROOT, "tensor_transformer_layer_amd", "libtpshard.so")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # A CPU-only checkout has no built library yet: build it here (hipcc cross-compiles for gfx950).
    # A GPU run never builds: the library must already be in the tree, or the imports fail loudly.
    if not os.path.exists(LIB) and shutil.which("hipcc") and not os.path.exists("/dev/kfd"):
        _load_build_module().build()


def _load_build_module():
    # by file path: importing it through the package would load the (missing or stale) library first
    import importlib.util
    path = os.path.join(ROOT, "tensor_transformer_layer_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_tp_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod
