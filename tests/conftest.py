import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def lib():
    """The HIP library binding (loads the in-tree libqlora.so, building it
    first only if no built library is present)."""
    so = os.path.join(ROOT, "parameter_efficient_fine_nf4_amd", "libqlora.so")
    if not os.path.exists(so):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_qlora_build", os.path.join(ROOT, "parameter_efficient_fine_nf4_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import parameter_efficient_fine_nf4_amd as q
    return q
