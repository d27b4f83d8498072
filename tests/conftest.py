import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU oracle time)")


def pytest_collection_modifyitems(config, items):
    # GPU tests first-class only where a GPU exists; on a CPU-only host they are
    # selected out by -m "not gpu" and, if run anyway, skip cleanly.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
