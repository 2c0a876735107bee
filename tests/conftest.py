import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def ls():
    """The HIP library binding.  On a machine with a GPU a missing library is an
    error, never a skip."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    import top_sparse_attention_ls_amd as lsmod
    lsmod.load()
    return lsmod


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name the case on stderr (flushed) before a GPU test touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write("\n[gpu case] %s\n" % request.node.nodeid)
        sys.stderr.flush()
    yield
