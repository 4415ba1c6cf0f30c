"""Build libaxonscan.so in-tree: the HIP kernels with hipcc for gfx950, the C-ABI layer with g++;
and libaxonmicro.so, the instruction and bandwidth microbenchmarks.

Usage: python -m selective_state_space_depthwise_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libaxonscan.so")
# Microbenchmarks of the instructions the kernels are built from (bench.py --micro); a library
# of its own so the product library carries none of it.
MICRO_SOURCE = "axon_microbench.hip"
MICRO_LIB = os.path.join(PKG, "libaxonmicro.so")

HIP_SOURCES = ["axon_kernels.hip", "axon_rowscan.hip", "axon_chanscan.hip", "axon_layer.hip",
               "axon_ssd.hip"]
CXX_SOURCES = ["axonscan_api.cpp"]
ARCH = "gfx950"
ROCM_LIB = "/opt/rocm/lib"  # hipBLASLt (the layer's projection GEMMs)
# Packed-FP32 instructions stay off: the compiler would otherwise form v_pk_* FP32 ops on its own.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libaxonscan)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link libaxonscan.so next to this file. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
              "-o", obj], verbose)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC,
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs,
          f"-L{ROCM_LIB}", "-lhipblaslt", f"-Wl,-rpath,{ROCM_LIB}"], verbose)
    os.replace(tmp, LIB)
    tmp = MICRO_LIB + f".tmp{os.getpid()}"
    _run([hipcc, *HIP_FLAGS, "-shared", "-I", CSRC, os.path.join(CSRC, MICRO_SOURCE), "-o", tmp],
         verbose)
    os.replace(tmp, MICRO_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
