"""Builds libmlip.so (the HIP library behind include/mlip.h) for gfx950.

Run ``python -m element_routed_moe_amd.build``.  Objects go to ``_build/``
(git-ignored); the shared library is written next to this file so that it
travels with the source tree.

``--debug-bounds`` builds the same sources with -DMLIP_DEBUG_BOUNDS into
libmlip_debug.so: every data-dependent index the kernels dereference is
checked against its range and a violation is printed (see common.h).  Load
it by setting MLIP_LIBRARY to its path before importing the binding.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmlip.so")
LIB_DEBUG = os.path.join(PKG, "libmlip_debug.so")
ARCH = "gfx950"

# Packed float32 VALU instructions are switched off for all device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, debug_bounds: bool = False) -> str:
    outdir = os.path.join(BUILD, "debug") if debug_bounds else BUILD
    obj = os.path.join(outdir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *(["-DMLIP_DEBUG_BOUNDS"] if debug_bounds else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(verbose: bool = True, debug_bounds: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, "debug") if debug_bounds else BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, debug_bounds), srcs))
    lib = LIB_DEBUG if debug_bounds else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build_library(debug_bounds="--debug-bounds" in sys.argv[1:])
    sys.exit(0)
