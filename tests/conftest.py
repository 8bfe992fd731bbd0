import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The worst |gpu - oracle| / bound of every bound-checked gradient, test by test."""
    try:
        from helpers import BOUND_RATIOS
    except ImportError:
        return
    if not BOUND_RATIOS:
        return
    terminalreporter.write_sep("-", "worst |gpu - oracle| / bound")
    for key in sorted(BOUND_RATIOS):
        terminalreporter.write_line(f"{BOUND_RATIOS[key]:.3f}  {key}")
    terminalreporter.write_line(f"{max(BOUND_RATIOS.values()):.3f}  overall worst")
