"""Build libpa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m paged_kv_cache_14_amd.build`` or ``build_library()``.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_PATH = os.path.join(PKG_DIR, "libpa.so")

ARCH = "gfx950"
# Packed fp32 VALU ops are left to none of our code: the feature is switched
# off for the device compile (hipcc's host pass warns it does not know it).
# -fno-honor-nans: no value the kernels compute arithmetic on can be NaN
# (slots that may hold NaN are replaced by selection before any use), so the
# compiler need not quiet every max operand (it otherwise spends one
# v_max_f32 per matrix-core result doing so).
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-honor-nans",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + \
        [os.path.join(CSRC, n) for n in ("pa_api.cpp", "block_manager.cpp", "check_batch.cpp")]


def build_library(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source into ``libpa.so`` next to this file; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}",
           "-x", "hip", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


ASAN_DIR = os.path.join(PKG_DIR, "_asan")
ASAN_LIB_PATH = os.path.join(ASAN_DIR, "libpa_asan.so")


def build_asan_library(verbose: bool = False) -> str:
    """The library with its host code built under AddressSanitizer
    (``_asan/libpa_asan.so``), for exercising the C ABI's validation,
    planning, block manager and batch check on the CPU.  The device code is
    compiled as usual (the host side needs its kernel objects to link) and
    never runs there.  A program that loads this library must itself be
    linked with -fsanitize=address: the ASan runtime lives in the program."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(ASAN_DIR, exist_ok=True)
    flags = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-honor-nans",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed ({res.returncode}):\n{res.stdout}\n"
                               f"{res.stderr}")

    objs = [os.path.join(ASAN_DIR, os.path.basename(src) + ".o") for src in sources()]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        list(pool.map(run, [[hipcc(), *flags, "-x", "hip", "-c", src, "-o", obj]
                            for src, obj in zip(sources(), objs)]))
    tmp = ASAN_LIB_PATH + ".tmp"
    run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-Xarch_host", "-fsanitize=address",
         *objs, "-o", tmp])
    os.replace(tmp, ASAN_LIB_PATH)
    for obj in objs:
        os.remove(obj)
    return ASAN_LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
