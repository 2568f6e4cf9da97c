import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print every error the parity checks measured (value against its bar), so a run's
    log carries the numbers and not only pass/fail.  The full-size workload rows come
    last."""
    try:
        from lora_cases import MEASURED
    except ImportError:
        return
    if not MEASURED:
        return
    tr = terminalreporter
    tr.write_line("")
    tr.write_line(f"measured errors ({len(MEASURED)} checks; value <= bar passes)")
    rows = sorted(MEASURED, key=lambda r: ("test_workload" in r[0], r[0]))
    for test, what, measure, value, bar in rows:
        name = test.split("::")[-1]
        tr.write_line(f"  {value:10.3e} <= {bar:7.1e}  {measure:12s}  {name}  {what}")
