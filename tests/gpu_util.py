"""Helpers for GPU tests: move seeded workloads to the device, run the HIP path, compare."""
import numpy as np

import workloads


def to_device_kv(wl, device="cuda"):
    import torch
    ks, vs = wl.kv_storage()
    if wl.dtype == "bf16":
        k = torch.from_numpy(np.ascontiguousarray(ks)).view(torch.bfloat16).to(device)
        v = torch.from_numpy(np.ascontiguousarray(vs)).view(torch.bfloat16).to(device)
    else:
        k = torch.from_numpy(np.ascontiguousarray(ks)).to(device)
        v = torch.from_numpy(np.ascontiguousarray(vs)).to(device)
    w = torch.from_numpy(np.ascontiguousarray(wl.w)).to(device)
    u = torch.from_numpy(np.ascontiguousarray(wl.u)).to(device)
    return k, v, w, u


def f64(a):
    return np.asarray(a, dtype=np.float64)


def seam_rows(T, chunk=128, every=256, max_seams=32):
    """Token rows for sampled summation-form checks: regular samples, both ends, and both sides
    of (up to max_seams, evenly spread) chunk seams."""
    rows = set(range(0, T, every)) | set(range(min(T, 4))) | set(range(max(0, T - 4), T))
    seams = list(range(chunk, T, chunk))
    stride = max(1, len(seams) // max_seams)
    for s in seams[::stride]:
        rows |= {s - 1, s}
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int64)


__all__ = ["to_device_kv", "f64", "seam_rows", "workloads"]
