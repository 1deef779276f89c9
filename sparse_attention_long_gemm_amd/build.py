"""Build libdsa.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m sparse_attention_long_gemm_amd.build          # or build_library() from Python

Objects go to sparse_attention_long_gemm_amd/_build/ (git-ignored); the shared library to
sparse_attention_long_gemm_amd/libdsa.so, which the Python binding loads.
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
LIB = os.path.join(PKG, "libdsa.so")

SOURCES = ["dsa_api.cpp", "indexer_topk.hip", "sparse_mqa.hip", "cache_write.hip",
           "ceilings.hip"]
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")

# Packed-fp32 VALU ops are switched off for all device code (see the design notes).
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build the DSA HIP library")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), f"--offload-arch={ARCH}", *COMMON, *lang, "-c", os.path.join(CSRC, src),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
