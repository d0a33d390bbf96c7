"""GPU parity of the Bi-WKV backward's launch forms (biwkv_backward through the C ABI) against the
float64 oracle's gradients of Eq. (5), with the scaled-error bar of test_gpu_backward.py (1e-4):

* the single launch, which exchanges both rounds' chunk sums between the chunks of a row while
  they run (the default for rows of several 128-token chunks that fit on the device);
* the multi-launch form (OPT_TWO_PASS = 1): chunk sums, carries and the two sweeps in separate
  launches, nothing waits;
* the fallback: with a poll limit of 0 (OPT_SPIN_LIMIT = 0) every wait of the single launch runs
  out at once, every row of several chunks is marked and computed again by one workgroup that
  needs no other; the stream's fault flags report it, and the results still hold the bar.
Each form is deterministic; the default form leaves the fault flags clear.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import f64, to_device_kv

pytestmark = pytest.mark.gpu

FORMS = ["single", "multi", "fallback"]
SHAPES = [  # (B, T, C, dtype): several chunks per row, ragged last chunk and tile, both dtypes
    (2, 700, 66, "bf16"),
    (1, 1025, 130, "f32"),
    (3, 129, 64, "bf16"),
    (1, 2000, 64, "f32"),
]


def _opts(form):
    import linear_complexity_vision_amd as L
    if form == "multi":
        return [(L.OPT_TWO_PASS, 1)]
    if form == "fallback":
        return [(L.OPT_SPIN_LIMIT, 0)]
    return []


def _run(wl, gy, form):
    import contextlib

    import torch

    import linear_complexity_vision_amd as L
    k, v, w, u = to_device_kv(wl)
    gd = torch.from_numpy(gy).cuda()
    with contextlib.ExitStack() as st:
        for o, val in _opts(form):
            st.enter_context(L.option(o, val))
        L.stream_fault_flags()  # clears the flags of earlier calls
        out = L.biwkv_backward(k, v, w, u, gd)
        torch.cuda.synchronize()
        flags = L.stream_fault_flags()
    return [x.cpu().numpy() for x in out], flags


def _scaled_err(got, ref, scale):
    return float(np.max(np.abs(got.astype(np.float64) - ref) / np.maximum(scale, 1e-30)))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("B,T,C,dtype", SHAPES)
def test_backward_form_matches_oracle(B, T, C, dtype, form):
    wl = workloads.make_random(400 + T + C, B, T, C, dtype=dtype, w_range=6.0, k_std=1.5, u_std=1.5)
    gy = np.random.Generator(np.random.PCG64(401 + T)).standard_normal(wl.k.shape).astype(np.float32)
    print(f"[case] backward form {form} {wl.name}", flush=True)
    got, flags = _run(wl, gy, form)
    ref = oracle.biwkv_backward_sum(f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u), f64(gy), with_scale=True)
    for name, x, r, s in zip(("dk", "dv", "dw", "du"), got, ref[:4], ref[4:]):
        assert np.isfinite(x).all(), name
        err = _scaled_err(x, r, s)
        print(f"[parity] backward {form} {wl.name} {name}: scaled error {err:.3e}", flush=True)
        assert err <= 1e-4, (name, err)
    if form == "fallback":
        assert flags != 0, "the fallback did not report itself"
    else:
        assert flags == 0, "a wait ran out"
    again, _ = _run(wl, gy, form)
    for a, b in zip(got, again):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("form", FORMS)
def test_backward_form_wide_rows(form):
    """A tile with w = -1e4 (wide form) next to an ordinary one, over several chunks per row."""
    wl = workloads.make_random(411, 2, 900, 128, dtype="bf16", w_range=5.0, k_std=1.5)
    w = wl.w.copy()
    w[70] = -1e4
    wl.w = w
    gy = np.random.Generator(np.random.PCG64(412)).standard_normal(wl.k.shape).astype(np.float32)
    print(f"[case] backward form {form} wide rows", flush=True)
    got, _ = _run(wl, gy, form)
    ref = oracle.biwkv_backward_sum(f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u), f64(gy), with_scale=True)
    tol = max(1e-4, 4.0 * float(np.abs(w).max()) * np.log2(np.e) * 2.0 ** -24)
    for name, x, r, s in zip(("dk", "dv", "dw", "du"), got, ref[:4], ref[4:]):
        err = _scaled_err(x, r, s)
        print(f"[parity] backward {form} wide rows {name}: scaled error {err:.3e}", flush=True)
        assert err <= tol, (name, err)
