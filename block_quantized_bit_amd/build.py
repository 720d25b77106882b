"""Build libwq.so (HIP, gfx950) in-tree with hipcc.

    python -m block_quantized_bit_amd.build

quant.hip and act.hip (bit-exact quantizers) are compiled with -ffp-contract=off so
no multiply-add is fused; every HIP file is compiled with packed-fp32 ops
disabled.  gemm.hip is compiled with LLVM's iterative ILP machine scheduler: with
it the register allocator keeps the GEMM accumulators in place across the K loop
instead of moving them between accumulation registers every iteration, and every
GEMM kernel but the 128 x 256 NVFP4 one runs faster (measured on MI355X); that one
is built from gemm_nvfp4_wide.hip with the default scheduler.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwq.so")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Wno-unused-command-line-argument"]

SOURCES = [
    ("quant.hip", ["-ffp-contract=off"]),
    ("act.hip", ["-ffp-contract=off"]),
    ("gemv.hip", []),
    ("gemm.hip", ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]),
    ("gemm_nvfp4_wide.hip", []),
    ("wq_api.cpp", ["-x", "hip"]),
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def _compile(src_flags):
    src, flags = src_flags
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
