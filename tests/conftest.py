import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse a tests/golden/*.txt fixture: 'key: row ; row' lines, '#' comments."""
    import numpy as np
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            rows = [[float(t) for t in r.split()] for r in val.split(";")]
            arr = np.array(rows, dtype=np.float64)
            out[key.strip()] = arr[0] if arr.shape[0] == 1 else arr
    return out
