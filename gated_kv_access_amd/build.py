"""Builds liboda.so, the C-ABI library of the ODA decode path, for gfx950.

oda_api.cpp (validation, planning, launch order) is plain host C++ and is
compiled with g++; oda_kernels.hip is compiled with hipcc for gfx950; the two
objects are linked by hipcc into gated_kv_access_amd/liboda.so.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liboda.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of every HIP object.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-I", INCLUDE, "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


PHASES_LIB = os.path.join(PKG, "liboda_phases.so")


def build(verbose: bool = False, extra_hip_flags=(), phases: bool = False) -> str:
    """Builds liboda.so, or with phases=True the profiling build
    liboda_phases.so (the same library with phase stamps, include/oda_phases.h)."""
    os.makedirs(BUILD, exist_ok=True)
    tag = "_phases" if phases else ""
    flags = ["-DODA_PHASE_STAMPS"] if phases else []
    api_o = os.path.join(BUILD, f"oda_api{tag}.o")
    ker_o = os.path.join(BUILD, f"oda_kernels{tag}.o")
    lib = PHASES_LIB if phases else LIB
    _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "oda_api.cpp"), "-o", api_o], verbose)
    _run([HIPCC, *HIP_FLAGS, *flags, *extra_hip_flags, "-c", os.path.join(CSRC, "oda_kernels.hip"), "-o", ker_o],
         verbose)
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, api_o, ker_o], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, phases=True)
    sys.exit(0)
