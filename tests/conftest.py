import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


if os.environ.get("RAXLORA_EXPECT_INDEX_CHECKS") == "1":
    import pytest

    @pytest.fixture(autouse=True)
    def _no_failed_index_checks(request):
        """Running on the index-checking build (tests/test_gpu_index_checks.py): every GPU
        test starts with the counts cleared and must leave no failed check behind."""
        if request.node.get_closest_marker("gpu") is None:
            yield
            return
        import rank_adapter_gemm_build_amd as rx
        enabled, _ = rx.index_checks(reset=True)
        assert enabled, f"{rx.LIB_PATH} is not the index-checking build"
        yield
        _, faults = rx.index_checks(reset=True)
        assert faults == 0, f"{faults} index checks failed in {request.node.nodeid}"


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
