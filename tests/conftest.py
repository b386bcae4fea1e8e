import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")


def load_golden(name):
    """Parse a tests/golden/*.txt fixture: '#' comments, then 'key v1 v2 ...' lines."""
    import numpy as np

    fields = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            fields[key] = vals
    M, N, K = (int(fields[k][0]) for k in ("M", "N", "K"))
    A = np.array([float(v) for v in fields["A"]], dtype=np.float32).reshape(M, N)
    B = np.array([float(v) for v in fields["B"]], dtype=np.float32).reshape(N, K)
    C = np.array([float(v) for v in fields["C"]], dtype=np.float64).reshape(M, K)
    return M, N, K, A, B, C


GOLDEN_FILES = ["leetgpu_example1.txt", "leetgpu_example2.txt", "tutorial_2x3x2.txt"]
