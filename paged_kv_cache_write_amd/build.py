"""Build libpa.so (HIP kernels for gfx950 + host C++) in-tree with hipcc.

Usage: python -m paged_kv_cache_write_amd.build [--verbose]
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
# the same sources with PA_DEBUG: device checks of slots, block ids and copy pairs
BUILD_DEBUG = os.path.join(ROOT, "_build_debug")
LIB_DEBUG = os.path.join(PKG, "libpa_debug.so")

SOURCES = ["decode.hip", "prefill.hip", "cache_ops.hip", "measure.hip", "block_manager.cpp",
           "capi.cpp", "engine.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _common():
    return ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall",
            "-Wno-unused-function"]


def _device_flags():
    # Packed-FP32 instructions are switched off for the device code; hipcc's
    # host pass warns that it does not know the feature, which is harmless.
    return [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops"]


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DEBUG if debug else BUILD, src + ".o")
    cmd = [hipcc(), "-c", path, "-o", obj] + _common() + (["-DPA_DEBUG"] if debug else [])
    if src.endswith(".hip"):
        cmd += ["-x", "hip"] + _device_flags()
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def _build_one(verbose: bool, debug: bool) -> str:
    os.makedirs(BUILD_DEBUG if debug else BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, debug), SOURCES))
    lib = LIB_DEBUG if debug else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every source and link libpa.so and libpa_debug.so; returns the
    path of libpa.so."""
    _build_one(verbose, debug=True)
    return _build_one(verbose, debug=False)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
