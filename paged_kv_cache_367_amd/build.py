"""Build libpa.so (the paged-attention C-ABI library) for gfx950 with hipcc.

Usage: python -m paged_kv_cache_367_amd.build [-v]

Every source is compiled for gfx950 only. Packed fp32 vector instructions are disabled
(-target-feature -packed-fp32-ops); hipcc's host pass warns that it does not know the
feature, which is harmless. Objects go to _build/ at the repository root; the library
is written next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
LIB = os.path.join(PKG, "libpa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["csrc/pa_api.cpp", "csrc/pa_decode.hip", "csrc/pa_prefill.hip",
           "csrc/pa_cache_ops.hip", "csrc/pa_block_manager.cpp", "csrc/pa_measure.hip"]
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose and (r.stdout or r.stderr):
        sys.stderr.write(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stderr}")
    return r


def compile_source(src: str, verbose: bool = False, extra=()) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    _run([HIPCC, *COMMON, *extra, "-x", "hip", "-c", os.path.join(PKG, src), "-o", obj], verbose)
    return obj


# Per-source flags. The prefill kernel keeps its MFMA accumulators in ordinary VGPRs
# (no accumulator-register copies around the vector-ALU rescale; 2 waves per SIMD fit).
EXTRA = {"csrc/pa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    """Compile every source and link libpa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: compile_source(s, verbose, EXTRA.get(s, ())), SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
