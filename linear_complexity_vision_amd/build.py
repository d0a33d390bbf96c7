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
CSRC = os.path.join(PKG, "csrc")
# the library's translation units (compiled at once, then linked into one shared library)
SOURCES = ["biwkv.hip", "fwd_f32.hip", "fwd_bf16.hip", "fwd_bf16_pair.hip", "bwd.hip"]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbiwkv.so")
# measurement only: streaming kernels with the forward's byte mix (a memory ceiling for the bench)
CEILING_SRC = os.path.join(CSRC, "hbm_ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libhbmceiling.so")
ARCH = "gfx950"
# -amdgpu-atomic-optimizer-strategy=None: the library's atomics are single-lane counters; the
# optimizer's wave-aggregated form reads an atomic's result right after issuing it, which would
# make the tile kernel's retirement count wait a full round trip before its sweeps.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def _hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def compile_command(src: str, obj: str, extra: list[str] | None = None) -> list[str]:
    return [_hipcc(), f"--offload-arch={ARCH}"] + FLAGS + ["-I", INCLUDE, "-c", "-o", obj, src] + (extra or [])


def hipcc_command(out: str = CEILING_LIB, extra: list[str] | None = None, src: str = CEILING_SRC) -> list[str]:
    """One-step compile and link of a single-file shared library."""
    return [_hipcc(), f"--offload-arch={ARCH}"] + FLAGS + ["-shared", "-I", INCLUDE, "-o", out, src] + (extra or [])


def build(verbose: bool = False, build_dir: str | None = None) -> str:
    """Compile both libraries (always recompiles; every translation unit at once) and return the
    path of libbiwkv.so."""
    bdir = build_dir or os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    jobs = []
    objs = []
    for name in SOURCES:
        obj = os.path.join(bdir, name.replace(".hip", ".o"))
        cmd = compile_command(os.path.join(CSRC, name), obj)
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        jobs.append((subprocess.Popen(cmd), name))
        objs.append(obj)
    cmd = hipcc_command(CEILING_LIB + ".tmp")
    jobs.append((subprocess.Popen(cmd), "hbm_ceiling.hip"))
    failed = [name for proc, name in jobs if proc.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, "hipcc", f"failed to compile {failed}")
    link = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(link), file=sys.stderr)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    os.replace(CEILING_LIB + ".tmp", CEILING_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
