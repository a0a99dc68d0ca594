import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_built():
    """Build the CPU-side libraries only when nothing is built yet."""
    import oracle
    import synth

    if not os.path.exists(oracle.LIB):
        from oracle import build as ob
        ob.build()
    if not os.path.exists(synth.HOST_LIB):
        from synth import build as sb
        sb.build_host()


_ensure_built()


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(1234)
