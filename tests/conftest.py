import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _ensure_built():
    """Build libgva.so once if it is missing (tests load what is built)."""
    lib = os.path.join(ROOT, "compressed_kv_cache_amd", "libgva.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "gva_build", os.path.join(ROOT, "compressed_kv_cache_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def pytest_configure(config):
    _ensure_built()
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built libgva")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    if not gpu_available():
        pytest.skip("no GPU visible")
    import torch
    return torch.device("cuda:0")
