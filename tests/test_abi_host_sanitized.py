"""The host-side argument validation of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The library's sources built with both sanitizers on the host code
(``build.py --sanitized``, the device code unchanged) are loaded in a child
process with the sanitizer runtime preloaded, and the host ABI tests run
against it; any report aborts the child (halt_on_error), so the test fails.
No call reaches the GPU: every case in those tests is rejected or finished
before any HIP call."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "_build", "sanitized", "libdspark_sanitized.so")


def test_host_abi_under_asan_and_ubsan():
    if not os.path.exists(SAN_LIB):
        pytest.skip("sanitized library not built (python semi_autoregressive_block_amd/build.py --sanitized)")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no AddressSanitizer runtime found")
    env = dict(os.environ, DSPARK_LIB_PATH=SAN_LIB, LD_PRELOAD=rt[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
