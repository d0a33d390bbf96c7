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
# measurement only: streaming kernels with the forward's byte mix (a memory ceiling for the bench)
CEILING_SRC = os.path.join(PKG, "csrc", "hbm_ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libhbmceiling.so")
ARCH = "gfx950"


def hipcc_command(out: str = LIB, extra: list[str] | None = None, src: str = SRC) -> list[str]:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-o", out, src] + (extra or [])


def _compile(src: str, lib: str, verbose: bool) -> subprocess.Popen:
    cmd = hipcc_command(lib + ".tmp", src=src)
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    return subprocess.Popen(cmd)


def build(verbose: bool = False) -> str:
    """Compile both libraries (always recompiles; the two compile at once) and return the path of
    libbiwkv.so."""
    jobs = [(_compile(SRC, LIB, verbose), LIB), (_compile(CEILING_SRC, CEILING_LIB, verbose), CEILING_LIB)]
    failed = [lib for proc, lib in jobs if proc.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, "hipcc", f"failed to build {failed}")
    for _, lib in jobs:
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
