import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


@pytest.fixture(scope="session", autouse=True)
def _built_library():
    """Build the HIP library in-tree when it is absent (hipcc cross-compiles
    for gfx950 without a GPU).  A present library is used as it is."""
    lib = os.path.join(ROOT, "paged_gqa_kv_amd", "libkvs.so")
    if not os.path.exists(lib) and os.path.exists("/opt/rocm/bin/hipcc"):
        from paged_gqa_kv_amd import build
        build.build()
    yield
