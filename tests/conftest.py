import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_sessionfinish(session, exitstatus):
    """With ASTR_PARITY_REPORT set, write the measured max-abs / max-rel of every GPU parity check."""
    path = os.environ.get("ASTR_PARITY_REPORT")
    helpers = sys.modules.get("_gpu_helpers")
    if not path or helpers is None or not helpers.PARITY_RECORDS:
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(helpers.PARITY_RECORDS, fh, indent=0)
