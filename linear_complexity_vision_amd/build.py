"""Builds libbiwkv.so (HIP, gfx950) in-tree with hipcc.

Packed-FP32 instructions are disabled for the device code (-packed-fp32-ops): the kernels are
plain scalar FP32 and must not be turned into v_pk_* by the compiler.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "biwkv.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbiwkv.so")
ARCH = "gfx950"


def hipcc_command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-o", out, SRC] + (extra or [])


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
