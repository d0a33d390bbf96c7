"""GPU parity of the Eq. (2) gate fused into Bi-WKV (biwkv_gated_forward, through the C ABI)
against the float64 oracle sigmoid(r) * Bi-WKV(k, v). Bar: R3 <= 1e-4 with the oracle's scale
multiplied by the gate (bf16 values are exact in the oracle).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import f64, to_device_kv
from tests.metrics import r3

pytestmark = pytest.mark.gpu


def _gate_input(wl, seed, scale=3.0):
    g = np.random.Generator(np.random.PCG64(seed))
    r = (g.standard_normal(wl.k.shape) * scale).astype(np.float32)
    if wl.dtype == "bf16":
        r = workloads._to_bf16_values(r)
    return r


def _run(wl, r):
    import torch

    import linear_complexity_vision_amd as L
    k, v, w, u = to_device_kv(wl)
    if wl.dtype == "bf16":
        rs = workloads.round_to_bf16_bits(r)
        rd = torch.from_numpy(np.ascontiguousarray(rs)).view(torch.bfloat16).cuda()
    else:
        rd = torch.from_numpy(np.ascontiguousarray(r)).cuda()
    y = L.biwkv_gated_forward(k, v, rd, w, u)
    torch.cuda.synchronize()
    assert L.stream_fault_flags() == 0
    return y.cpu().numpy()


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_gated_workload_shapes(index):
    wl = workloads.make(index)
    r = _gate_input(wl, 500 + index)
    print(f"[case] biwkv_gated_forward {wl.name}", flush=True)
    y = _run(wl, r)
    assert np.isfinite(y).all()
    y_ref, s_ref = oracle.biwkv_gated(f64(wl.k), f64(wl.v), f64(r), f64(wl.w), f64(wl.u), with_scale=True)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] gated {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C", [(1, 1, 4), (2, 3, 6), (1, 129, 66), (2, 255, 130), (3, 200, 100),
                                   (1, 700, 1), (1, 1025, 64), (2, 2047, 66), (1, 3000, 130)])
def test_gated_edge_shapes(B, T, C, dtype):
    wl = workloads.make_random(23 + T + C, B, T, C, dtype=dtype, w_range=8.0, k_std=3.0, u_std=2.0)
    r = _gate_input(wl, 600 + T + C, scale=6.0)
    r.reshape(-1)[:3] = [60.0, -60.0, 0.0][: r.size]  # saturated gates and the midpoint
    print(f"[case] biwkv_gated_forward edge {wl.name}", flush=True)
    y = _run(wl, r)
    y_ref, s_ref = oracle.biwkv_gated(f64(wl.k), f64(wl.v), f64(r), f64(wl.w), f64(wl.u), with_scale=True)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] gated edge {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


def test_gated_wide_form():
    wl = workloads.make_random(41, 1, 2500, 64, dtype="f32", w_range=5.0)
    wl.w = wl.w.copy()
    wl.w[0::3] = -1e4
    r = _gate_input(wl, 41)
    print("[case] biwkv_gated_forward wide", flush=True)
    y = _run(wl, r)
    assert np.isfinite(y).all()
    # the summation form: the RNN form's lam^T leaves float64 at |w| = 1e4
    y_ref, s_ref = oracle.biwkv_gated(f64(wl.k), f64(wl.v), f64(r), f64(wl.w), f64(wl.u), with_scale=True,
                                      use_sum=True)
    tol = 1e-4  # the wide form's exact token counts hold the plain bar at |w| = 1e4
    assert r3(y, y_ref, s_ref) <= tol
