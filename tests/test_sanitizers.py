"""CPU sanitizer run: the host planner and C ABI (g++ with AddressSanitizer and
UndefinedBehaviorSanitizer, linked with the ordinary device objects) and the C
oracle (gcc, same sanitizers) run the planner, ABI and oracle-pin tests in a
child pytest with the sanitizer runtimes preloaded.  Any out-of-bounds access,
use after free or undefined behaviour aborts the child and fails this test.
Leak checking is off: the Python interpreter itself is not instrumented."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.slow


def _runtime(name):
    try:
        p = subprocess.check_output(["gcc", "-print-file-name=" + name], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_planner_and_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from dimensional_sparse_local_amd import build as nb
    import oracle

    na_lib = nb.build_host_sanitized(str(tmp_path / "san" / "libna.so"))
    or_lib = oracle.build_sanitized(str(tmp_path / "san" / "liboracle.so"))
    maps = str(tmp_path / "maps.txt")
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan + " " + ubsan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:allocator_may_return_null=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "NA_TEST_LIBRARY": na_lib,
        "ORACLE_TEST_LIBRARY": or_lib,
        "NA_TEST_MAPS_OUT": maps,
    })
    tests = ["tests/test_planner.py", "tests/test_abi.py", "tests/test_oracle_pins.py",
             "tests/test_oracle_backward_pins.py", "tests/test_oracle_pi_pins.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + tests, cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    mapped = open(maps).read()
    assert na_lib in mapped and or_lib in mapped, "the sanitizer builds were not the ones loaded"
