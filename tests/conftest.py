import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large host-side work (minutes)")


def _gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    # GPU tests are selected with -m gpu on a machine with a GPU.  If they are collected on
    # a host without a GPU they fail loudly rather than being skipped silently,
    # unless the marker expression deselects them.
    pass


@pytest.fixture(scope="session")
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a visible GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library (built in-tree first if nothing is there)."""
    import dense_gemm_work_amd as dg

    return dg
