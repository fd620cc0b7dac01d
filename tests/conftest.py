import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libnvfp4")


def read_golden(name):
    """Parse a `key = value` golden file (comments start with #)."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals = [float(t) for t in v.split()]
            out[k] = vals if len(vals) > 1 else vals[0]
    return out


@pytest.fixture
def golden():
    return read_golden
