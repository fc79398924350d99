import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workloads")


def _ensure_built():
    """Tests load what is built; they build only when nothing is there."""
    import importlib
    lib = os.path.join(ROOT, "computation_collective_amd", "libhocf.so")
    if not os.path.exists(lib):
        importlib.import_module("computation_collective_amd.build").build()
    olib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(olib):
        importlib.import_module("oracle.build").build()


_ensure_built()


def pytest_runtest_logreport(report):
    """If HOCF_FAILURE_LOG names a file, append each failure's details to it as
    it happens, so they survive a run that is cut short."""
    path = os.environ.get("HOCF_FAILURE_LOG")
    if report.failed and path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(f"==== {report.nodeid} ({report.when})\n{report.longreprtext}\n")
