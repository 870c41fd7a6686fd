import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes)")


def _oracle_stale():
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    src = os.path.join(ROOT, "oracle", "mx_oracle.c")
    return (not os.path.exists(lib)) or os.path.getmtime(lib) < os.path.getmtime(src)


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built from source here if it is missing or stale)."""
    import oracle
    if _oracle_stale():
        from oracle import build
        build.build()
    return oracle.default()
