"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

build.py --sanitize compiles the host code (argument and table checks, packer and
validator, shared-decode planner, cos/sin tables, cache simulator) with
g++ -fsanitize=address,undefined and no device code; the CPU tests of that
layer then run against it in a child process with the sanitizer runtime
preloaded.  Any sanitizer report aborts the child (UBSan without recovery).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_layer_is_clean_under_asan_and_ubsan():
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    asan = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime on this machine")
    b = subprocess.run([sys.executable, os.path.join(ROOT, "position_agnostic_kv_lazy_amd", "build.py"),
                        "--sanitize"], capture_output=True, text=True, cwd=ROOT, timeout=600)
    assert b.returncode == 0, b.stdout + b.stderr
    lib = os.path.join(ROOT, "position_agnostic_kv_lazy_amd", "_build", "sanitize",
                       "liblazyattn_sanitized.so")
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", LAZYATTN_LIB=lib)
    t = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_cache_sim.py", "tests/test_shared_plan.py",
                        "tests/test_check_tables.py"],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=900)
    out = t.stdout + t.stderr
    assert t.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
