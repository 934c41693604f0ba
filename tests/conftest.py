import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_terminal_summary(terminalreporter):
    """The largest parity errors the GPU tests observed, against their bounds."""
    gc = sys.modules.get("gpu_common")
    worst = getattr(gc, "WORST", None) if gc else None
    if not worst:
        return
    terminalreporter.write_line("parity, largest errors observed (value / bound, where):")
    for name in sorted(worst):
        v, bnd, where = worst[name]
        terminalreporter.write_line(f"  {name}: {v:.3e} / {bnd:.0e} ({where})")
