import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# The oracle mutation test runs this suite against a planted-mistake copy of
# the oracle placed in the directory this variable names.
_MUT = os.environ.get("TT_ORACLE_MUTANT_DIR")
if _MUT:
    sys.path.insert(0, _MUT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def rel_l2(a, ref):
    """||a - ref||_2 / ||ref||_2 in float64 (absolute norm when ref is all zero)."""
    import numpy as np
    a = np.asarray(a, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    d = np.linalg.norm(a - ref)
    n = np.linalg.norm(ref)
    return float(d / n) if n > 0 else float(d)


@pytest.fixture
def golden():
    import json

    def load(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)
    return load
