"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
argument validation over extreme shapes (no 32-bit product may overflow),
workspace arithmetic, and the host helpers writing into exactly sized
buffers (tests/sanitize/abi_checks.cpp).  Host code only: no kernel is
launched."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))

pytestmark = pytest.mark.skipif(not shutil.which("hipcc") and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def test_abi_checks_under_asan_and_ubsan():
    import build as B
    exe = B.build()
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr[-3000:])
    assert r.returncode == 0, r.stderr[-3000:]
    assert "abi checks passed" in r.stdout
