import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test (oracle at large sizes)")


def gpu_available() -> bool:
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
    return torch.device("cuda", 0)


def _ensure_library():
    """Build libtrimul.so only when nothing is built (normally build() ran first)."""
    lib = os.path.join(ROOT, "triangle_multiplicative_update_amd", "libtrimul.so")
    if not os.path.exists(lib):
        import importlib.util
        path = os.path.join(ROOT, "triangle_multiplicative_update_amd", "build.py")
        spec = importlib.util.spec_from_file_location("_trimul_build", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


_ensure_library()
