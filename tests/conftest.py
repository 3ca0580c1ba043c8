import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def lib_path():
    """Path of the built C-ABI library; builds it once if nothing is built yet."""
    from tiled_attention_12_amd import _build
    path = _build.library_path()
    if not os.path.exists(path):
        import __graft_entry__
        __graft_entry__.build()
    return path
