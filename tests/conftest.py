import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases that take tens of seconds")


def pytest_collection_modifyitems(config, items):
    """GPU tests need a visible GPU; without one (a CPU-only host) they are skipped.
    On a GPU host a missing library is an error, never a skip."""
    import pytest

    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
