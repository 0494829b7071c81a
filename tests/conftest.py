import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libsmla")


def _ensure_built():
    """Tests load the built library; build it only when none is there."""
    lib = os.path.join(ROOT, "sparse_mla_attention_resolve_amd", "libsmla.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_smla_build", os.path.join(ROOT, "sparse_mla_attention_resolve_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


_ensure_built()
