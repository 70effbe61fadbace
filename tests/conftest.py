import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of host work)")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; on a host without one they are skipped, not failed,
    # unless they were explicitly selected with -m gpu (then they must run).
    import importlib.util
    has_torch = importlib.util.find_spec("torch") is not None
    gpu = False
    if has_torch:
        import torch
        gpu = torch.cuda.is_available()
    markexpr = config.getoption("-m") or ""
    if gpu or "gpu" in markexpr and "not gpu" not in markexpr:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
