"""The host validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU): api.cpp and paley.cpp are built with g++
and the sanitizers (kernel launchers stubbed out), and tests/test_abi_host.py
runs against that library in a child process with the ASan runtime
preloaded.  Any sanitizer report aborts the child and fails this test."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_abi_host_under_asan_ubsan():
    import build_hostsan as B
    lib = B.build()
    rt = B.asan_runtime()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("g++ has no shared AddressSanitizer runtime")
    env = dict(os.environ)
    env.update(HADAROT_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_host.py")], env=env, capture_output=True, text=True,
                       cwd=os.path.dirname(HERE), timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
