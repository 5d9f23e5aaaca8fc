import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    config.addinivalue_line("markers", "device_code: calls the library's device entry points (host-side "
                                       "checks only, no GPU needed); needs the full library, not the "
                                       "host-only sanitizer build")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped when no GPU is visible, so a CPU-only run of the
    # whole suite stays green; on a GPU machine they run.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # name the case on stderr before any GPU work starts, so a run that dies
    # mid-test still says which case it was
    if "gpu" in request.keywords:
        sys.stderr.write(f"\n[gpu-case] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield
