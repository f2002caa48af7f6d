import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def load_golden(name):
    """Parse a hand-worked fixture: ``key = rows`` with rows split by ';'."""
    import numpy as np
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#") or "=" not in line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            rows = [[float(v) for v in r.split()] for r in val.split(";")]
            out[key] = np.array(rows if len(rows) > 1 else rows[0], dtype=np.float64)
    return out


@pytest.fixture
def golden():
    return load_golden
