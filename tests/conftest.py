import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Observed attention errors against their tolerances (GPU parity runs)."""
    gu = sys.modules.get("gpu_util")
    if gu is None or not getattr(gu, "OBSERVED", None):
        return
    terminalreporter.write_sep("-", "attention outputs: largest max-abs error per test (tolerance)")
    for test, (err, tol) in sorted(gu.OBSERVED.items()):
        terminalreporter.write_line(f"{err:10.3e}  ({tol:g}, {100.0 * err / tol:5.1f}% used)  {test}")
