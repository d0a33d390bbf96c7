"""Seeded synthetic inputs for the Bi-WKV / Q-Shift path (shared by tests, bench and smoke).

This module holds no arithmetic of the method: it only draws random numbers and rounds them to
the storage formats. Both the HIP path and the CPU oracle consume exactly the arrays made here.

Recipe: ``numpy.random.Generator(PCG64(seed))`` with seed = workload index; float64 draws, rounded
to float32 (round-to-nearest-even), then to bfloat16 (round-to-nearest-even) where a workload
stores k and v as bf16. Draw order is x (Q-Shift workload only), k, v, w, u.

The five workloads stand in for the pages' image-token workloads (the Vision-RWKV article's
ImageNet 224px setting gives 196 tokens; its efficiency study scales inputs to 2048px, i.e. 16384
tokens at patch 16). Real k and v would be projections of images through trained weights; none
are available, so iid normals are used, with w and k ranges chosen to stress stability.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def round_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even; NaN stays NaN."""
    bits = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    nan = np.isnan(x32)
    rounded = np.where(nan, (bits >> 16) | 0x40, rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b16: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(b16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    B: int
    H: int
    W: int
    C: int
    dtype: str                      # "f32" or "bf16": storage type of k and v
    k: np.ndarray                   # float32 values (bf16-exact when dtype == "bf16")
    v: np.ndarray
    w: np.ndarray                   # float32 [C]
    u: np.ndarray                   # float32 [C]
    x: np.ndarray | None = None     # float32 Q-Shift input (Q-Shift workload only)
    shift: int = 1
    gamma: float = 0.25
    notes: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.H * self.W

    def kv_storage(self):
        """k and v in their storage format: float32 arrays, or uint16 bf16 bit patterns."""
        if self.dtype == "bf16":
            return round_to_bf16_bits(self.k), round_to_bf16_bits(self.v)
        return self.k, self.v


def _normal(rng, shape, std=1.0):
    return (rng.standard_normal(size=shape) * std).astype(np.float32)


def _uniform(rng, lo, hi, n):
    return rng.uniform(lo, hi, size=n).astype(np.float32)


def _to_bf16_values(x32):
    return bf16_bits_to_f32(round_to_bf16_bits(x32))


# name: (B, H, W, C, dtype, w range, k std, u std, has x)
SPECS = {
    1: ("biwkv_B1_T196_C192_f32", 1, 14, 14, 192, "f32", 3.0, 1.0, 1.0, False),
    2: ("qshift_biwkv_B64_T196_C384_f32", 64, 14, 14, 384, "f32", 3.0, 1.0, 1.0, True),
    3: ("biwkv_B32_T784_C768_bf16", 32, 28, 28, 768, "bf16", 5.0, 1.0, 1.0, False),
    4: ("biwkv_qshift_B4_T4096_C1024_bf16", 4, 64, 64, 1024, "bf16", 5.0, 1.0, 1.0, False),
    5: ("biwkv_B1_T16384_C768_f32_stress", 1, 128, 128, 768, "f32", 8.0, 4.0, 3.0, False),
}


def make(index: int) -> Workload:
    """The five seeded workloads (index 1..5), at their full sizes."""
    name, B, H, W, C, dtype, wr, kstd, ustd, has_x = SPECS[index]
    rng = np.random.Generator(np.random.PCG64(index))
    T = H * W
    x = _normal(rng, (B, T, C)) if has_x else None
    k = _normal(rng, (B, T, C), kstd)
    v = _normal(rng, (B, T, C))
    w = _uniform(rng, -wr, wr, C)
    u = _normal(rng, (C,), ustd)
    if index == 5:
        w[0::8] = 0.0  # exact zeros in one channel of every eight
    if dtype == "bf16":
        k, v = _to_bf16_values(k), _to_bf16_values(v)
    return Workload(name, B, H, W, C, dtype, k, v, w, u, x=x, shift=1, gamma=0.25,
                    notes={"seed": index})


def make_random(seed: int, B: int, T: int, C: int, dtype: str = "f32", w_range: float = 5.0,
                k_std: float = 1.0, u_std: float = 1.0, H: int | None = None, W: int | None = None) -> Workload:
    """A seeded random workload of any shape (edge and ragged cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if H is None or W is None:
        H, W = 1, T
    assert H * W == T
    k = _normal(rng, (B, T, C), k_std)
    v = _normal(rng, (B, T, C))
    w = _uniform(rng, -w_range, w_range, C)
    u = _normal(rng, (C,), u_std)
    if dtype == "bf16":
        k, v = _to_bf16_values(k), _to_bf16_values(v)
    return Workload(f"random_s{seed}_B{B}_T{T}_C{C}_{dtype}", B, H, W, C, dtype, k, v, w, u,
                    notes={"seed": seed})


# Sparse (MAE-masked) inputs: the visible tokens of an image with 75% of its patches masked (MAE's
# usual ratio; the article follows ViT's MAE setting). Only the visible tokens are present, N of
# them per image; k, v, w, u are drawn as for the dense workloads (iid, so any subset of tokens has
# the same distribution).
# name: (seed, B, N, C, dtype, w range)
MAE_SPECS = {
    1: ("mae_B64_N49_C384_f32", 6, 64, 49, 384, "f32", 3.0),        # 25% of a 14 x 14 grid
    2: ("mae_B16_N1024_C1024_bf16", 7, 16, 1024, 1024, "bf16", 5.0),  # 25% of 64 x 64; B * N * C as
                                                                       # for 4 x 4096 x 1024
}


def make_mae(index: int) -> Workload:
    """The sparse-input workloads of the bidirectional shift (shift 1, gamma 1/4)."""
    name, seed, B, N, C, dtype, wr = MAE_SPECS[index]
    wl = make_random(seed, B, N, C, dtype=dtype, w_range=wr)
    wl.name = name
    return wl
