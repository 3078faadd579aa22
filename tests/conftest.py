import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


_HAS_GPU = None


def _has_gpu():
    global _HAS_GPU
    if _HAS_GPU is None:
        try:
            import torch
            _HAS_GPU = bool(torch.cuda.is_available())
        except Exception:
            _HAS_GPU = False
    return _HAS_GPU


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped only where no GPU exists at all; on a GPU machine
    # they run and fail loudly if the HIP library is missing.
    gpu_items = [it for it in items if "gpu" in it.keywords]
    if gpu_items and not _has_gpu():
        skip = pytest.mark.skip(reason="no GPU visible")
        for it in gpu_items:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()
