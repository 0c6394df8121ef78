import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _lib_path():
    return os.path.join(ROOT, "paged_kv_cache_378_amd", "libpa.so")


@pytest.fixture(scope="session")
def libpa():
    """The built C-ABI library (builds it once if nothing is built yet)."""
    if not os.path.exists(_lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    from paged_kv_cache_378_amd import _lib
    return _lib


@pytest.fixture(scope="session")
def gpu(libpa):
    import torch
    if not torch.cuda.is_available():
        # GPU tests never pass silently on a machine without a GPU.
        pytest.fail("tests marked gpu need a visible GPU (run them with -m gpu on the GPU host)")
    return torch.device("cuda:0")
