import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU oracle work (full-size sampled parity)")


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    return torch.cuda.is_available()


def pytest_sessionfinish(session, exitstatus):
    """Write the band counts the GPU tests recorded (strict / explained / fail per case)."""
    gu = sys.modules.get("gpu_util")
    if gu is None or not (getattr(gu, "RECORDS", None) or getattr(gu, "REPORTS", None)):
        return
    import json
    # MOE_PARITY_RECORDS names the file (default: parity_out/parity_records.json)
    path = os.environ.get("MOE_PARITY_RECORDS") or os.path.join(ROOT, "parity_out", "parity_records.json")
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as fh:
        json.dump({"exitstatus": int(exitstatus), "records": gu.RECORDS, "reports": gu.REPORTS}, fh, indent=1)
