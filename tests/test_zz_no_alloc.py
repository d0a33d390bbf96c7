"""The allocation-free forward (biwkv_forward_noalloc, through the C ABI) against biwkv_forward.

Both run the same kernels on the same inputs and fold the chunks' sums in the same order, so the
outputs must be equal bit for bit: on two calls in a row, the second with a smaller input (the
static scratch keeps the first call's contents), in one launch and in two, and the oracle bar
(R3 <= 1e-4) holds for both. A problem whose chunk sums exceed the static buffer is refused
before anything is enqueued. Runs alone in a fresh process as well as after the other tests.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import f64, to_device_kv
from tests.metrics import r3

pytestmark = pytest.mark.gpu


def _noalloc(L, k, v, w, u, out, dtype):
    import torch
    B, T, C = k.shape
    return L.load_library().biwkv_forward_noalloc(
        k.data_ptr(), v.data_ptr(), w.data_ptr(), u.data_ptr(), out.data_ptr(), B, T, C, dtype,
        torch.cuda.current_stream().cuda_stream)


def _check(L, wl):
    import torch
    k, v, w, u = to_device_kv(wl)
    dt = L.BF16 if wl.dtype == "bf16" else L.F32
    out = torch.full(k.shape, float("nan"), dtype=torch.float32, device=k.device)
    assert _noalloc(L, k, v, w, u, out, dt) == 0
    ref = L.biwkv_forward(k, v, w, u)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got, ref.cpu().numpy())
    y_ref, s_ref = oracle.biwkv_rnn(f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u), with_scale=True)
    err = r3(got, y_ref, s_ref)
    print(f"[parity] noalloc {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


def test_noalloc_matches_forward_on_two_calls_large_then_small():
    import linear_complexity_vision_amd as L
    print("[case] noalloc: config 4 (one launch, 512 chunks), then a smaller row set", flush=True)
    _check(L, workloads.make(4))
    _check(L, workloads.make_random(91, 1, 2000, 130, dtype="bf16", w_range=6.0))


def test_noalloc_two_launch_rows_and_single_chunk_rows():
    import linear_complexity_vision_amd as L
    print("[case] noalloc: config 5 (one launch over 1.5 residency rounds, then the two-pass form), "
          "then single-chunk rows", flush=True)
    _check(L, workloads.make(5))
    with L.option(L.OPT_TWO_PASS, 1):
        _check(L, workloads.make(5))
    _check(L, workloads.make_random(92, 3, 300, 100, dtype="f32", w_range=5.0))
    with L.option(L.OPT_TWO_PASS, 1):
        _check(L, workloads.make_random(93, 2, 3000, 128, dtype="bf16", w_range=5.0))


def test_noalloc_refuses_beyond_its_buffer():
    """B = 32, T = 16384, C = 1024 bf16 needs 32 * 16 * 128 chunks of 4 KiB (256 MiB) in the
    two-pass form: refused before any launch (the pointers are never used)."""
    import torch

    import linear_complexity_vision_amd as L
    lib = L.load_library()
    x = torch.empty(16, dtype=torch.float32, device="cuda")
    p = x.data_ptr()
    rc = lib.biwkv_forward_noalloc(p, p + 0x100000000, p + 0x200000000, p + 0x200001000, p + 0x300000000,
                                   32, 16384, 1024, L.BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == L.status_codes()["BIWKV_ERR_SCRATCH"]
    assert "static buffer" in L.status_string(rc)
