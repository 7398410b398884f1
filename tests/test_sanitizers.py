"""The host-side suite under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the HIP library with sanitized host code (every -fsanitize flag after
-Xarch_host; the device code is built as usual) and the fp64 oracle with the
same sanitizers, then runs the CPU tests that exercise them -- the ABI's
argument checks, plans and status codes, and the oracle with all its pins --
in a child process with the clang ASan runtime preloaded. Any sanitizer
report, or any failing test, fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SUITE = ["tests/test_abi.py", "tests/test_oracle_pins.py", "tests/test_oracle_gates.py",
         "tests/test_oracle_bwd.py", "tests/test_check_pins.py"]


@pytest.mark.timeout(900)
def test_host_suite_under_asan_and_ubsan():
    from block_sparse_long_moba_amd import build
    import oracle
    lib = build.build_sanitized(OUT)
    olib = oracle.build_sanitized(OUT)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": build.asan_runtime(),
        "LD_LIBRARY_PATH": "/opt/rocm/llvm/lib:" + env.get("LD_LIBRARY_PATH", ""),
        # Python itself is not instrumented and keeps memory until exit
        "ASAN_OPTIONS": "detect_leaks=0",
        "UBSAN_OPTIONS": "print_stacktrace=1",
        "MOBA_LIBRARY": lib,
        "MOBA_ORACLE_LIBRARY": olib,
    })
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-m", "not gpu",
                        "-p", "no:faulthandler", "-p", "no:cacheprovider"] + SUITE,
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=840)
    out = p.stdout
    for marker in ("runtime error:", "ERROR: AddressSanitizer", "SUMMARY: "):
        assert marker not in out, out[-4000:]
    assert p.returncode == 0, out[-4000:]
    assert " passed" in out and " failed" not in out, out[-2000:]
