import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_host_libs():
    """Build the generator and the oracle if nothing is built yet (gcc, seconds)."""
    import synth
    import oracle
    if not os.path.exists(synth.LIB_PATH):
        from synth import build as sb
        sb.build()
    if not os.path.exists(oracle.LIB_PATH):
        from oracle import build as ob
        ob.build()


_ensure_host_libs()
