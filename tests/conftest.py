import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def _ensure_library():
    lib = os.path.join(ROOT, "long_context_sparse_page_amd", "liblocks.so")
    if not os.path.exists(lib):
        from long_context_sparse_page_amd import build_lib
        build_lib.build()


_ensure_library()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible GPU")
    return torch.device("cuda:0")
