"""The host code of the C ABI -- descriptor, packed-weight layout and the
workspace planner, whose carve is size_t offset arithmetic -- under
AddressSanitizer and UndefinedBehaviorSanitizer: the library is rebuilt with
rnn_api.cpp instrumented (device code unchanged) and the CPU boundary tests
run against it in a child process with the ASan runtime preloaded.  Needs no
GPU."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.slow

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(1200)
def test_boundary_tests_under_asan_and_ubsan():
    from layer_rnn_forward_amd import build as b
    if not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not available")
    rt = b.asan_runtime()
    if not (os.path.isabs(rt) and os.path.exists(rt)):
        pytest.skip("no shared ASan runtime next to the compiler")
    lib = b.build_sanitized()
    env = dict(os.environ, RNN_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary_cpu.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
