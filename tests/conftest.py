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


def pytest_terminal_summary(terminalreporter):
    """Per GPU test file: how many elements the plain 1e-5 * T bound judged,
    how many missed it, and the worst ratio (tests/gpu_util.py)."""
    gu = sys.modules.get("gpu_util")
    if gu is None or not gu.PLAIN_STATS:
        return
    terminalreporter.write_sep("-", "plain-bound tally per file")
    for f, st in sorted(gu.PLAIN_STATS.items()):
        terminalreporter.write_line(
            "%-34s elements %10d  beyond plain %6d  worst plain ratio %.3g%s" % (
                f, st["elements"], st["beyond_plain"], st["worst_plain_ratio"],
                "  (group term allowed)" if st["group_term"] else ""))
