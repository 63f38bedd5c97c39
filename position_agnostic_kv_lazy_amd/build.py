"""Build liblazyattn.so in-tree with hipcc for gfx950.

    python position_agnostic_kv_lazy_amd/build.py

(run as a script: importing the package loads the library being rebuilt).

Every HIP source is compiled with -Xclang -target-feature -Xclang
-packed-fp32-ops, so the device compiler never emits packed fp32 arithmetic;
the host pass prints a harmless "not a recognized feature" warning for it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblazyattn.so")

SOURCES = ["lazy_attn_host.cpp", "decode_split.cpp", "attn_f32.hip", "decode_bf16.hip",
           "decode_shared_bf16.hip", "prefill_bf16.hip", "store_kv.hip", "cache_sim.cpp"]
# host-only build with AddressSanitizer + UndefinedBehaviorSanitizer (no device code)
SANITIZE_SOURCES = ["lazy_attn_host.cpp", "decode_split.cpp", "cache_sim.cpp", "host_only_stubs.cpp"]
SANITIZE_LIB = os.path.join(BUILD, "sanitize", "liblazyattn_sanitized.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = os.environ.get("LAZYATTN_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """Host layer only, g++ with -fsanitize=address,undefined, for CPU tests.

    Load it with the sanitizer runtime preloaded, e.g.
        LD_PRELOAD=$(g++ -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
        LAZYATTN_LIB=position_agnostic_kv_lazy_amd/_build/sanitize/liblazyattn_sanitized.so \
        python -m pytest tests/test_abi.py tests/test_cache_sim.py tests/test_shared_plan.py
    (tests/test_sanitized_host.py runs exactly that).
    """
    out = os.path.dirname(SANITIZE_LIB)
    os.makedirs(out, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fvisibility=hidden", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", CSRC, "-I", os.path.join(ROCM, "include")]
    cmd += [os.path.join(CSRC, f) for f in SANITIZE_SOURCES]
    cmd += ["-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"),
            "-lamdhip64", "-lpthread", "-o", SANITIZE_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SANITIZE_LIB}")
    return SANITIZE_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
