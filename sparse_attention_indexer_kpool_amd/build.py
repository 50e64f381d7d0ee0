"""Build libkpool.so (hand-written HIP kernels for gfx950 + the C ABI) in the
package directory with hipcc. Usage: python -m sparse_attention_indexer_kpool_amd.build"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkpool.so")

SOURCES = ["api.cpp", "check.hip", "compress.hip", "decode.hip", "expand.hip", "fp8_quant.hip", "logits.hip",
           "mla.hip", "proj.hip", "select.hip"]

ARCH = "gfx950"
FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # packed FP32 VALU forms stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, out: str = LIB, defines=()) -> str:
    """Compile every source and link `out`. `defines` (e.g. ["-DNAME=1"]) are
    extra preprocessor definitions for variant builds."""
    build_dir = BUILD if out == LIB else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 6)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, tuple(defines)), SOURCES))
    LIBOUT = out
    tmp = LIBOUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIBOUT)
    if verbose:
        print(f"built {LIBOUT}")
    return LIBOUT


if __name__ == "__main__":
    build()
    sys.exit(0)
