import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def rel_fro(got, want) -> float:
    """Relative Frobenius error ||got - want||_F / ||want||_F (float64)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want.ravel())
    num = np.linalg.norm((got - want).ravel())
    return float(num / den) if den > 0 else float(num)


@pytest.fixture
def rng():
    return np.random.Generator(np.random.PCG64(20191001))
