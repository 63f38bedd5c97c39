"""The boundary is a C ABI: a plain C99 program (tests/c/abi_host_calls.c)
includes include/lazy_attn.h, links liblazyattn.so with gcc and calls the
host entry points (tables, packer, validator, shared-decode planner,
workspace size, cache simulator) with no Python or C++ in between."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "position_agnostic_kv_lazy_amd")


def test_plain_c_caller(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(LIBDIR, "liblazyattn.so")):
        pytest.skip("library not built")
    exe = tmp_path / "abi_host_calls"
    b = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "abi_host_calls.c"), "-o", str(exe),
                        "-L", LIBDIR, "-llazyattn", f"-Wl,-rpath,{LIBDIR}"],
                       capture_output=True, text=True, timeout=120)
    assert b.returncode == 0, b.stdout + b.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
