import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: full-size workloads (minutes of CPU oracle time)")


@pytest.fixture(autouse=True)
def _progress_log(request):
    """Append each test's id to $QMA_PROGRESS_LOG before it runs, so a run
    that dies on the GPU still names the case it was in."""
    path = os.environ.get("QMA_PROGRESS_LOG")
    if path:
        with open(path, "a") as f:
            f.write(f"START {request.node.nodeid}\n")
            f.flush()
    yield
    if path:
        with open(path, "a") as f:
            f.write(f"END   {request.node.nodeid}\n")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_moe_align_amd import qma
    qma.lib()               # fails loudly when the HIP library is missing
    return torch.device("cuda:0")
