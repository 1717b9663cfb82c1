import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Worst |gpu - oracle| / tolerance of every parity test that compared outputs
    (1.0 is the bar), so that a run shows how much margin is left."""
    from tests.harness import MARGINS
    if not MARGINS:
        return
    terminalreporter.write_sep("-", "parity margins: worst |gpu - oracle| / (2e-3 + 1e-2 |oracle|)")
    for name, r in sorted(MARGINS.items(), key=lambda kv: -kv[1]):
        terminalreporter.write_line(f"{r:8.4f}  {name}")
