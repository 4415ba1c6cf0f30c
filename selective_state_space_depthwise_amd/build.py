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
               "axon_ssd.hip", "axon_noalloc.hip"]
CXX_SOURCES = ["axonscan_api.cpp"]
ARCH = "gfx950"
ROCM_LIB = "/opt/rocm/lib"  # hipBLASLt (the layer's projection GEMMs)
# Packed-FP32 instructions stay off: the compiler would otherwise form v_pk_* FP32 ops on its own.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument"]


# Sanitizer build (host code only; the GPU code is built as usual): AddressSanitizer and
# UndefinedBehaviorSanitizer in the C-ABI layer, the host side of the HIP sources and the CPU
# oracle, all with the ROCm clang so that one sanitizer runtime serves them all.
SAN_DIR = os.path.join(PKG, "_build", "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libaxonscan.so")
SAN_ORACLE = os.path.join(SAN_DIR, "libaxon_oracle.so")
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]
CLANG = "/opt/rocm/llvm/bin/clang"


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime (preloaded into the Python that loads the libraries)."""
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                         capture_output=True, text=True).stdout.strip()
    if not os.path.exists(out):
        import glob

        cands = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not cands:
            raise RuntimeError("clang's AddressSanitizer runtime was not found")
        out = cands[0]
    return out


def build_sanitized(verbose: bool = False) -> dict:
    """Build libaxonscan.so and the oracle with ASan + UBSan into _build/sanitize; returns the
    environment that runs the CPU tests against them."""
    os.makedirs(SAN_DIR, exist_ok=True)
    hipcc = _hipcc()
    host_san = [f for flag in SAN_FLAGS for f in ("-Xarch_host", flag)]
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(SAN_DIR, src.replace(".hip", ".o"))
        _run([hipcc, *HIP_FLAGS, *host_san, "-I", INCLUDE, "-I", CSRC, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(SAN_DIR, src.replace(".cpp", ".o"))
        _run([CLANG + "++", "-O1", "-std=c++17", "-fPIC", "-Wall", *SAN_FLAGS, "-I", INCLUDE,
              "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-shared-libasan",
          *host_san, "-o", SAN_LIB, *objs, f"-L{ROCM_LIB}", "-lhipblaslt",
          f"-Wl,-rpath,{ROCM_LIB}"], verbose)
    oracle_src = os.path.join(ROOT, "oracle", "axon_oracle.c")
    _run([CLANG, "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-shared-libasan",
          *SAN_FLAGS, "-o", SAN_ORACLE, oracle_src, "-lm", "-lpthread"], verbose)
    return {"LD_PRELOAD": asan_runtime(), "AXONSCAN_LIB": SAN_LIB, "AXON_ORACLE_LIB": SAN_ORACLE,
            "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


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
    if "--sanitize" in sys.argv:
        # python -m selective_state_space_depthwise_amd.build --sanitize [--run-tests]
        env = build_sanitized(verbose="-q" not in sys.argv)
        print(" ".join(f"{k}={v}" for k, v in env.items()))
        if "--run-tests" in sys.argv:
            full = dict(os.environ, **env)
            rc = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"),
                                 "-q", "-m", "not gpu", "-p", "no:cacheprovider"],
                                env=full).returncode
            sys.exit(rc)
    else:
        print(build(verbose="-q" not in sys.argv))
