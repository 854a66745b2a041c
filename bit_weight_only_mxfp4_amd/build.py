"""Build libtt.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_weight_only_mxfp4_amd.build

Every source is compiled for gfx950 only, without fast-math, with fp32
denormals kept, with packed-fp32 instruction selection switched off and with
the leading kernel arguments preloaded into scalar registers.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtt.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["abi.cpp", "pack.cpp", "mxfp4_gateup.hip", "int4_gemv.hip", "moe.hip", "fp8_gemv.hip", "attention.hip",
           "dequant.hip", "stream_read.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
         "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # the first 16 dwords of every kernel's arguments arrive in scalar
         # registers at wave launch instead of through a memory load
         "-mllvm", "-amdgpu-kernarg-preload-count=16",
         "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libtt.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libtt.so failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
