import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_sessionfinish(session, exitstatus):
    """Write the GEMM parity statistics the GPU tests recorded, if asked to."""
    path = os.environ.get("FP8Q_PARITY_REPORT")
    if not path:
        return
    try:
        import helpers
    except ImportError:
        return
    if helpers.PARITY_STATS:
        import json
        with open(path, "w") as f:
            json.dump(helpers.PARITY_STATS, f, indent=1)
