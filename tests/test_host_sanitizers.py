"""The host code of the library (quantizers, argument checks, status codes)
under AddressSanitizer and UndefinedBehaviorSanitizer: the library is rebuilt
with both on its host code, and the CPU tests of the C-ABI run against that
build in a child process with the sanitizer runtime preloaded.  Any report
aborts the child (no recovery), which fails this test."""
import os
import subprocess
import sys

from fp8_block_scaled_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_asan_and_ubsan(tmp_path):
    lib = build.build_host_sanitized(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms      # instrumented
    env = dict(os.environ, GFG_LIBRARY=lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
