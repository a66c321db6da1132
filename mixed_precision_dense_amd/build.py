"""Build the HIP library ``libmpgemm.so`` in-tree with hipcc for gfx950.

The translation units (the C-ABI argument checks, the dispatch code, one kernel unit per input
type or format pair, the split kernel of the three-product GEMM and the sparse kernels) are
compiled in parallel and linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmpgemm.so")
SOURCES = ["mpgemm_host.cpp", "mpgemm_api.hip", "kern_f16.hip", "kern_bf16.hip", "kern_i8.hip", "bf16x3.hip",
           "kern_fp8_fp8.hip", "kern_fp8_bf8.hip", "kern_bf8_fp8.hip", "kern_bf8_bf8.hip",
           "sp24.hip", "sp24_f16.hip", "sp24_bf16.hip", "sp24_i8.hip", "sp24_fp8_fp8.hip",
           "sp24_fp8_bf8.hip", "sp24_bf8_fp8.hip", "sp24_bf8_bf8.hip"]
ARCH = "gfx950"

# Packed FP32 instructions are kept out of all generated code.
COMMON_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-I" + INCLUDE, "-I" + CSRC]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmpgemm.so")


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libmpgemm.so``; returns its path."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
