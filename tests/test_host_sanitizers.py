"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): an instrumented copy of librkv.so runs the CPU tests of the ABI
(argument validation of every entry point, workspace sizes, state set-up),
the restart policy, the delay-token rule and the mel filterbank, with the
sanitizer runtime preloaded into a child Python; any report aborts it.  A
positive control (a host array one element shorter than the stream count
passed to rkv_state_init_host) must be caught as a heap buffer overflow, so
the instrumentation is known to be live."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = ["tests/test_abi.py", "tests/test_restart_policy.py", "tests/test_tcond_host.py",
         "tests/test_mel_host.py"]


@pytest.fixture(scope="module")
def sanitized():
    if not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("no hipcc")
    try:
        from rolling_window_kv_amd import build_host_sanitized as bhs
    except ImportError:
        pytest.skip("host-sanitizer build script not present")
    lib = bhs.build()
    env = dict(os.environ, RKV_LIBRARY=lib, LD_PRELOAD=bhs.runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_host_code_is_clean_under_asan_and_ubsan(sanitized):
    r = subprocess.run([sys.executable, "-m", "pytest", *TESTS, "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=sanitized,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out
    assert r.returncode == 0


def test_sanitizer_catches_a_short_host_array(sanitized):
    code = textwrap.dedent("""
        import ctypes
        import numpy as np
        from rolling_window_kv_amd import rkv
        S = 4
        cfg = rkv.make_cfg(S, 1, max_cap=375)
        win = np.full(S - 1, 375, np.int32)          # one element short
        cap = np.full(S, 375, np.int32)
        org = np.zeros(S, np.int64)
        st = np.zeros(S * rkv.STATE_DTYPE.itemsize, np.uint8)
        rkv.lib().rkv_state_init_host(ctypes.byref(cfg), win.ctypes.data, cap.ctypes.data,
                                      org.ctypes.data, st.ctypes.data)
        print("not caught")
    """)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized,
                       capture_output=True, text=True, timeout=120)
    out = r.stdout + r.stderr
    assert "heap-buffer-overflow" in out, out[-2000:]
    assert "not caught" not in out
