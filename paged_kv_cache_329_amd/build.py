"""Builds libpagedkv.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m paged_kv_cache_329_amd.build`` (or ``build()`` from Python).  Sources
are compiled in parallel into ``_build/`` at the repository root and linked into
``paged_kv_cache_329_amd/libpagedkv.so``.  Every HIP source is compiled with packed
fp32 instructions disabled.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["status.cpp", "allocator.cpp", "vmm.cpp", "cache_ops.hip", "attention_decode.hip", "attention_prefill.hip"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked at $HIPCC, /opt/rocm/bin/hipcc, PATH)")


COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [_hipcc(), *COMMON_FLAGS, *HIP_FLAGS, "-c", path, "-o", obj]
    else:
        rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
        cmd = [_hipcc(), "-x", "c++", *COMMON_FLAGS, "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include", "-c", path,
               "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    # The host pass does not know the device-only feature flag; that warning is harmless.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l).strip()
    if msgs and verbose:
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source and links the library; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
