"""The copy-ceiling kernels (libhbmceiling, used by bench.py for the memory ceiling of the
forward's byte mix) move what they claim: out = k + v element by element (one fp32 rounding, the
same as torch's fp32 add on the host), for every piece width, cache policy, unroll and a
grid-stride loop with a ragged tail; elements past n are left alone."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _lib():
    from linear_complexity_vision_amd import build
    if not os.path.exists(build.CEILING_LIB):
        pytest.fail("libhbmceiling.so is not built")
    f = ctypes.CDLL(build.CEILING_LIB).hbm_stream
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    f.restype = ctypes.c_int
    return f


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("policy", list(range(8)))
@pytest.mark.parametrize("blocks,unroll", [(0, 1), (37, 2), (5, 4)])
def test_stream_copies_sum(dtype, policy, blocks, unroll):
    import torch
    f = _lib()
    n = 4096 * 3 + 8
    g = torch.Generator().manual_seed(1000 + policy)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.randn(n, generator=g).to(tdt)
    v = torch.randn(n, generator=g).to(tdt)
    want = k.float() + v.float()
    kd, vd = k.cuda(), v.cuda()
    out = torch.full((n + 64,), -7.0, device="cuda")
    print(f"[case] hbm_stream {dtype} policy {policy} blocks {blocks} unroll {unroll}", flush=True)
    rc = f(kd.data_ptr(), vd.data_ptr(), out.data_ptr(), n, 1 if dtype == "bf16" else 0, 0, blocks, unroll,
           policy, None)
    assert rc == 0
    torch.cuda.synchronize()
    got = out.cpu()
    assert torch.equal(got[:n], want)
    assert bool((got[n:] == -7.0).all())
