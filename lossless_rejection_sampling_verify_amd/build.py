"""Compile the HIP library ``libspecverify.so`` for gfx950 with hipcc.

Packed fp32 instructions are disabled (``-packed-fp32-ops``) and floating-point
contraction is off, so every weight is computed with the same IEEE operations
wherever it appears.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "spec_verify.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libspecverify.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


DEMO_SRC = os.path.join(HERE, "csrc", "abi_demo.c")
DEMO_PATH = os.path.join(HERE, "abi_demo")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    build_demo(verbose)
    return LIB_PATH


def build_demo(verbose: bool = False) -> str:
    """The plain C consumer of the ABI (gcc, linked against the library next to it)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, "-o", DEMO_PATH + ".tmp", DEMO_SRC,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-L", HERE, "-lspecverify",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(DEMO_PATH + ".tmp", DEMO_PATH)
    return DEMO_PATH


if __name__ == "__main__":
    print(build(verbose=True))
