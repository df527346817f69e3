import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_sessionfinish(session, exitstatus):
    # Error figures of every parity comparison of the session (max-abs,
    # mean-abs, max-rel), written as JSON when ETA_PARITY_LOG names a file.
    path = os.environ.get("ETA_PARITY_LOG")
    if not path:
        return
    import parity
    d = os.path.dirname(path)
    if d:
        os.makedirs(d, exist_ok=True)
    with open(path, "w") as f:
        json.dump(parity.LOG, f, indent=0)


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    return torch.device("cuda", 0)
