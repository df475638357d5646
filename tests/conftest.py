import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU oracle comparison at full workload size")


def pytest_collection_modifyitems(config, items):
    # GPU tests on a machine without a GPU are skipped with a clear reason,
    # never silently routed anywhere else.
    try:
        import torch

        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
