import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running oracle check")


def pytest_sessionfinish(session, exitstatus):
    """Write the near-tie exemptions that the GPU parity tests recorded (test name ->
    exempt pairs, units that needed one, units checked) to $HGA_PARITY_RECORD, or to
    parity_exemptions.json in the run's output folder when that folder exists."""
    chk = sys.modules.get("tests.hga_check")
    if chk is None or not getattr(chk, "EXEMPTIONS", None):
        return
    path = os.environ.get("HGA_PARITY_RECORD")
    if not path and os.path.isdir(os.path.join(ROOT, "gpurun_out")):
        path = os.path.join(ROOT, "gpurun_out", "parity_exemptions.json")
    if path:
        with open(path, "w") as f:
            json.dump(chk.EXEMPTIONS, f, indent=1, sort_keys=True)
