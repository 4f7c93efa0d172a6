import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available():
    try:
        import torch
    except Exception:
        return False
    return torch.cuda.is_available()


def pytest_collection_modifyitems(config, items):
    # torch is imported only when a collected test needs the GPU
    if not any("gpu" in item.keywords for item in items) or gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
