"""The host planner built with AddressSanitizer and UndefinedBehaviorSanitizer
(no device code; HIP entry points stubbed), running the native-planner tests
in a subprocess: bit-exact plans of every standard workload and plan variant,
random and fuzzed trees, error codes, null pointers, device-image sizing and
the work-item rules.  Any out-of-bounds access, use after free or undefined
behaviour in the planner's index arithmetic aborts the run.  Host-only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the planner tests that need no GPU entry point
SUBSET = ("bit_exact or errors or null_pointer or device_bytes or wide_mfma_item_rule or launch_size or "
          "fuzzed or exports")


def _asan_runtime():
    if not shutil.which("g++"):
        return None
    path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(900)
def test_planner_under_address_and_ub_sanitizers():
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("g++ with the AddressSanitizer runtime is not available")
    sys.path.insert(0, ROOT)
    from tree_structured_decode_amd import build as B
    lib = B.build_planner_sanitized()
    env = dict(os.environ, DEFT_LIB_PATH=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONHASHSEED="0")
    env.pop("PYTEST_XDIST_WORKER", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-p", "no:xdist",
                        os.path.join(ROOT, "tests", "test_native_planner.py"), "-m", "not gpu", "-k", SUBSET],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=850)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
