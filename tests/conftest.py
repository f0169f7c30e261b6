import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _has_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def pytest_collection_modifyitems(config, items):
    # GPU tests are never silently skipped on a host with a GPU: if a gpu-marked test
    # is selected and no GPU is visible, it fails loudly inside the test via
    # the binding. On a CPU-only host they are skipped unless explicitly
    # requested with -m gpu.
    markexpr = config.getoption("-m") or ""
    if _has_gpu() or ("gpu" in markexpr and "not gpu" not in markexpr):
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
