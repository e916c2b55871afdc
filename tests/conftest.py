import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """How many compared units needed the fp32-resolution floor above the
    plain 1e-4 score bar (tests/checks.py)."""
    try:
        from checks import FLOOR_STATS
    except ImportError:
        return
    if FLOOR_STATS["units"]:
        terminalreporter.write_line(
            f"z-score floor: {FLOOR_STATS['above']} of {FLOOR_STATS['units']} compared units "
            f"needed one above 1e-4 (largest {FLOOR_STATS['max']:.2e})")
