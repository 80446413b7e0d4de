import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# The CPU sanitizer run (tests/test_sanitizers.py) starts pytest on the
# planner and oracle tests with sanitizer builds of both libraries.
if os.environ.get("NA_TEST_LIBRARY"):
    from dimensional_sparse_local_amd import na as _na

    _na._LIB_PATH = os.environ["NA_TEST_LIBRARY"]
if os.environ.get("ORACLE_TEST_LIBRARY"):
    import oracle as _oracle

    _oracle._LIB = os.environ["ORACLE_TEST_LIBRARY"]


def pytest_sessionfinish(session, exitstatus):
    # the sanitizer run records which shared libraries this process mapped
    out = os.environ.get("NA_TEST_MAPS_OUT")
    if out:
        with open("/proc/self/maps") as f, open(out, "w") as g:
            g.write(f.read())


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
