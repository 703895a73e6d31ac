import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running (full-size shapes)")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def tiny_shape():
    import workload
    return workload.config(0).shape


def pytest_runtest_logstart(nodeid, location):
    """Start of every test, also as a line in gpurun_out/pytest_progress.log
    when that folder exists (long GPU tests are otherwise silent under -q)."""
    _progress(f"start {nodeid}")


def pytest_runtest_logfinish(nodeid, location):
    _progress(f"end {nodeid}")


def _progress(line: str):
    import time
    d = os.path.join(ROOT, "gpurun_out")
    if os.path.isdir(d):
        with open(os.path.join(d, "pytest_progress.log"), "a") as f:
            f.write(f"{time.strftime('%H:%M:%S')} {line}\n")
