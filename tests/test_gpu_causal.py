"""GPU parity of the causal attention (biwkv_causal_forward, through the C ABI) against the CPU
float64 oracle's causal forms: Eq. (7) of the Vision-RWKV article without the backward states,
i.e. earlier tokens plus the bonus term. Bar: R3 <= 1e-4 (bf16 values are exact in the oracle).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import f64, to_device_kv
from tests.metrics import r3

pytestmark = pytest.mark.gpu


def _run(wl):
    import torch

    import linear_complexity_vision_amd as L
    k, v, w, u = to_device_kv(wl)
    y = L.biwkv_causal_forward(k, v, w, u)
    torch.cuda.synchronize()
    assert L.stream_fault_flags() == 0
    return y.cpu().numpy()


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_causal_workload_shapes(index):
    """The Bi-WKV workloads' shapes and value distributions, through the causal entry."""
    wl = workloads.make(index)
    print(f"[case] biwkv_causal_forward {wl.name}", flush=True)
    y = _run(wl)
    assert np.isfinite(y).all()
    y_ref, s_ref = oracle.biwkv_causal_rnn(f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u), with_scale=True)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] causal {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


CAUSAL_SHAPES = [(1, 1, 4), (2, 2, 6), (1, 3, 2), (1, 129, 66), (2, 255, 130), (1, 513, 64),
                 (3, 200, 100), (1, 700, 1), (2, 1000, 256),
                 # several chunks per row, ragged last chunk and tile
                 (1, 1025, 64), (2, 2047, 66), (1, 3000, 130), (1, 5121, 32)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C", CAUSAL_SHAPES)
def test_causal_edge_shapes(B, T, C, dtype):
    wl = workloads.make_random(11 + T + C, B, T, C, dtype=dtype, w_range=8.0, k_std=3.0, u_std=2.0)
    print(f"[case] biwkv_causal_forward edge {wl.name}", flush=True)
    y = _run(wl)
    y_ref, s_ref = oracle.biwkv_causal_sum(f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u), with_scale=True)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] causal edge {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


@pytest.mark.parametrize("T", [600, 2500])
@pytest.mark.parametrize("case", ["k_plus_100", "u_100", "w_plus_1e4", "w_minus_1e4", "w_mixed_wide",
                                  "k_row_start_far_below", "u_minus_41", "k_spread_40"])
def test_causal_extreme_values(case, T):
    """k_row_start_far_below: the row's first tokens carry keys 100 below the rest, so their
    outputs are weighted means of terms some 2^-144 below the lane's largest; u_minus_41 keeps the
    bonus (u log2 e = -59.2) inside the fast form's range."""
    wl = workloads.make_random(98, 1, T, 64, dtype="f32", w_range=5.0, k_std=1.0)
    k, w, u = wl.k.copy(), wl.w.copy(), wl.u.copy()
    if case == "k_plus_100":
        k += np.float32(100.0)
    elif case == "u_100":
        u[:] = 100.0
    elif case == "w_plus_1e4":
        w[:] = 1e4
    elif case == "w_minus_1e4":
        w[:] = -1e4
    elif case == "w_mixed_wide":
        w[0::3] = -1e4
        w[1::3] = 3e3
    elif case == "k_row_start_far_below":
        k[:, :3] -= np.float32(100.0)
    elif case == "u_minus_41":
        u[:] = -41.0
    elif case == "k_spread_40":
        k *= np.float32(10.0)
    wl.k, wl.w, wl.u = k, w, u
    print(f"[case] biwkv_causal_forward extreme {case} T={T}", flush=True)
    y = _run(wl)
    assert np.isfinite(y).all()
    y_ref, s_ref = oracle.biwkv_causal_sum(f64(k), f64(wl.v), f64(w), f64(u), with_scale=True)
    err = r3(y, y_ref, s_ref)
    tol = 1e-4  # the wide form's exact token counts hold the plain bar at |w| = 1e4
    print(f"[parity] causal extreme {case} T={T}: R3 = {err:.3e} (tol {tol:.1e})", flush=True)
    assert err <= tol


def test_causal_last_token_matches_bidirectional_and_runs_are_deterministic():
    import torch

    import linear_complexity_vision_amd as L
    wl = workloads.make_random(31, 2, 3000, 128, dtype="bf16")
    k, v, w, u = to_device_kv(wl)
    print("[case] causal vs bidirectional last token, determinism", flush=True)
    yc = L.biwkv_causal_forward(k, v, w, u)
    yb = L.biwkv_forward(k, v, w, u)
    torch.cuda.synchronize()
    np.testing.assert_allclose(yc[:, -1].cpu().numpy(), yb[:, -1].cpu().numpy(), rtol=1e-5, atol=1e-6)
    first = yc.cpu().numpy()
    for _ in range(5):
        np.testing.assert_array_equal(L.biwkv_causal_forward(k, v, w, u).cpu().numpy(), first)
    assert L.stream_fault_flags() == 0
