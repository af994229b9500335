"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/test_abi.py run in a child process against lib/libqsa_san.so (the same
sources, host code instrumented, device code unchanged) with the sanitizer
runtime preloaded.  No compute call is made, so no GPU is needed."""
import os
import subprocess
import sys

from learned_sparse_attention_qsa_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import os, sys
import learned_sparse_attention_qsa_amd as Q
assert Q.LIB_PATH == os.environ["QSA_LIBRARY"], Q.LIB_PATH
Q.load_library()
maps = open("/proc/self/maps").read()
assert "libqsa_san.so" in maps and "libclang_rt.asan" in maps, "sanitized library not loaded"
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", sys.argv[1],
                      "-k", "not fails_loudly_without_library"]))
"""


def test_abi_checks_run_clean_under_asan_and_ubsan():
    san = B.SAN_LIB
    if not os.path.exists(san):
        B.build_sanitized()
    env = dict(os.environ, QSA_LIBRARY=san, LD_PRELOAD=B.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", CHILD, os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout
