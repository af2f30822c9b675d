import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # A gpu-marked test on a machine without a GPU is skipped, never faked.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # Name the case on the real stderr before it touches the GPU, so a run
    # that ends the process still says which case it was in.
    if "gpu" in request.keywords:
        sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    import parity
    parity.CURRENT_TEST = request.node.nodeid
    yield
