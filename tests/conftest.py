import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is visible; on a CPU host they are skipped with a reason.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _no_expired_waits(request):
    """After every GPU test: no launch on the test's stream had a bounded wait between workgroups expire
    (ssd_workspace_check on every workspace the binding keeps for that stream)."""
    yield
    if "gpu" not in request.keywords:
        return
    import torch
    if not torch.cuda.is_available():
        return
    import selective_state_space_diag_amd as ssd
    ssd.workspace_check()
