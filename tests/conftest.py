import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if item.get_closest_marker("gpu"):
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # name the case on stderr (bypassing capture) before any GPU work, so a run that dies
    # inside a kernel still says which case it was
    if request.node.get_closest_marker("gpu"):
        print(f"[gpu-case] {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield
