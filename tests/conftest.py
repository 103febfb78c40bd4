import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _has_gpu_device() -> bool:
    return os.path.exists("/dev/kfd")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped only on a machine with no AMD GPU device node at all.
    # Where /dev/kfd exists they run, and fail loudly if the GPU or library is unusable.
    if _has_gpu_device():
        return
    skip = pytest.mark.skip(reason="no AMD GPU device on this machine")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
