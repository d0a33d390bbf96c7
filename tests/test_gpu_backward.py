"""GPU parity of the Bi-WKV backward (biwkv_backward, through the C ABI) against the float64
oracle's gradients of Eq. (5) (definition form with magnitude scales; linear-time form at the
workload sizes).

Metric: each gradient element's error over its scale, the oracle's sum of the magnitudes that make
it up (sum_t |g_t| p_ti for dv_i; sum_t |g_t| p_ti (|v_i| + |y_t|) for dk_i, and likewise for du and
dw), so cancellation between terms, or a difference v_i - y_t of two nearly equal values, does not
turn rounding into a large relative error. Bar: 1e-4, as for the forward pass.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import f64, to_device_kv

pytestmark = pytest.mark.gpu


def _upstream(wl, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal(wl.k.shape).astype(np.float32)


def _run(wl, gy):
    import torch

    import linear_complexity_vision_amd as L
    k, v, w, u = to_device_kv(wl)
    dk, dv, dw, du = L.biwkv_backward(k, v, w, u, torch.from_numpy(gy).cuda())
    torch.cuda.synchronize()
    return dk.cpu().numpy(), dv.cpu().numpy(), dw.cpu().numpy(), du.cpu().numpy()


def _scaled_err(got, ref, scale):
    return float(np.max(np.abs(got.astype(np.float64) - ref) / np.maximum(scale, 1e-30)))


def _check_against_sum(wl, gy, tol=1e-4, label=""):
    got = _run(wl, gy)
    ref = oracle.biwkv_backward_sum(f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u), f64(gy), with_scale=True)
    for name, x, r, s in zip(("dk", "dv", "dw", "du"), got, ref[:4], ref[4:]):
        assert np.isfinite(x).all(), name
        err = _scaled_err(x, r, s)
        print(f"[parity] backward {label} {name}: scaled error {err:.3e}", flush=True)
        assert err <= tol, (name, err)


BWD_SHAPES = [(1, 1, 4), (2, 2, 6), (1, 3, 2), (1, 8, 64), (1, 9, 66), (2, 129, 66), (1, 200, 100),
              (1, 513, 64), (2, 700, 3), (1, 1025, 130)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C", BWD_SHAPES)
def test_backward_edge_shapes(B, T, C, dtype):
    wl = workloads.make_random(61 + T + C, B, T, C, dtype=dtype, w_range=8.0, k_std=2.0, u_std=2.0)
    gy = _upstream(wl, 71 + T + C)
    print(f"[case] biwkv_backward edge {wl.name}", flush=True)
    _check_against_sum(wl, gy, label=wl.name)


@pytest.mark.parametrize("case", ["k_plus_100", "u_100", "w_plus_1e4", "w_minus_1e4", "w_zero"])
def test_backward_extreme_values(case):
    wl = workloads.make_random(97, 1, 600, 64, dtype="f32", w_range=5.0)
    k, w, u = wl.k.copy(), wl.w.copy(), wl.u.copy()
    if case == "k_plus_100":
        k += np.float32(100.0)
    elif case == "u_100":
        u[:] = 100.0
    elif case == "w_plus_1e4":
        w[:] = 1e4
    elif case == "w_minus_1e4":
        w[:] = -1e4
    elif case == "w_zero":
        w[:] = 0.0
    wl.k, wl.w, wl.u = k, w, u
    gy = _upstream(wl, 98)
    print(f"[case] biwkv_backward extreme {case}", flush=True)
    # same fp32 exponent-resolution bound as the forward extreme cases
    tol = max(1e-4, 4.0 * float(np.abs(w).max()) * np.log2(np.e) * 2.0 ** -24)
    _check_against_sum(wl, gy, tol=tol, label=case)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_mixed_forms_across_tiles(dtype):
    """Three 64-channel tiles: the middle one holds a channel with w = -1e4 (its tile takes the
    wide form), the others are ordinary (fast form); T = 1000 spans many chunks, so every stage of
    the call must take the same form per tile."""
    wl = workloads.make_random(123, 2, 1000, 192, dtype=dtype, w_range=5.0, k_std=1.5)
    w = wl.w.copy()
    w[70] = -1e4
    w[100] = 3e3
    wl.w = w
    gy = _upstream(wl, 124)
    print(f"[case] biwkv_backward mixed fast / wide tiles {dtype}", flush=True)
    tol = max(1e-4, 4.0 * float(np.abs(w).max()) * np.log2(np.e) * 2.0 ** -24)
    _check_against_sum(wl, gy, tol=tol, label=f"mixed tiles {dtype}")


@pytest.mark.parametrize("index", [1, 3, 4, 5])
def test_backward_workload_shapes(index):
    """Full-size workloads. dk and dv of every element against the linear-time oracle (pinned to the
    definition form on small sizes), with element scales sum_t |g_t| p_ti for dv_i and
    |v_i| sum_t |g_t| p_ti + sum_t |g_t y_t| p_ti for dk_i, from the same recurrences run on |g| and
    |g y|. dw and du (sums over every token and batch item) on a sample of channels against the
    definition form with its magnitude scales; the definition form holds a T x T matrix per thread,
    so it runs on a few threads."""
    wl = workloads.make(index)
    gy = _upstream(wl, 800 + index)
    print(f"[case] biwkv_backward {wl.name}", flush=True)
    dk, dv, dw, du = _run(wl, gy)
    k, v, w, u, g = f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u), f64(gy)
    rk, rv, _, _ = oracle.biwkv_backward_rnn(k, v, w, u, g)
    y = oracle.biwkv_rnn(k, v, w, u)
    sv = oracle.biwkv_backward_rnn(k, v, w, u, np.abs(g))[1]  # sum_t |g_t| p_ti
    scale_k = np.abs(v) * sv + np.abs(oracle.biwkv_backward_rnn(k, v, w, u, np.abs(g) * np.abs(y))[1])
    for name, x, r, s in (("dv", dv, rv, sv), ("dk", dk, rk, scale_k)):
        err = _scaled_err(x, r, s)
        print(f"[parity] backward {wl.name} {name}: scaled error {err:.3e}", flush=True)
        assert err <= 1e-4, (name, err)
    B, T, C = wl.k.shape
    cols = np.unique(np.linspace(0, C - 1, 8).round().astype(np.int64))
    threads = int(max(1, min(4, B * cols.size)))
    ref = oracle.biwkv_backward_sum(k[:, :, cols], v[:, :, cols], w[cols], u[cols], g[:, :, cols],
                                    with_scale=True, threads=threads)
    for name, x, r, s in (("dw", dw[cols], ref[2], ref[6]), ("du", du[cols], ref[3], ref[7])):
        err = _scaled_err(x, r, s)
        print(f"[parity] backward {wl.name} {name} (channels {cols.tolist()}): scaled error {err:.3e}",
              flush=True)
        assert err <= 1e-4, (name, err)


def test_backward_deterministic_and_identities():
    import torch

    import linear_complexity_vision_amd as L
    wl = workloads.make_random(55, 2, 3000, 128, dtype="bf16", w_range=6.0)
    gy = _upstream(wl, 56)
    k, v, w, u = to_device_kv(wl)
    gd = torch.from_numpy(gy).cuda()
    print("[case] backward determinism and identities", flush=True)
    first = [x.cpu().numpy() for x in L.biwkv_backward(k, v, w, u, gd)]
    for _ in range(3):
        again = [x.cpu().numpy() for x in L.biwkv_backward(k, v, w, u, gd)]
        for a, b in zip(first, again):
            np.testing.assert_array_equal(a, b)
    dk, dv = first[0].astype(np.float64), first[1].astype(np.float64)
    # sum_i dv_i = sum_t g_t and sum_i dk_i = 0 per (batch, channel)
    np.testing.assert_allclose(dv.sum(axis=1), gy.astype(np.float64).sum(axis=1), rtol=1e-4, atol=1e-3)
    assert np.abs(dk.sum(axis=1)).max() <= 1e-4 * np.abs(dk).sum(axis=1).max()


def test_backward_on_two_streams_matches_default_stream():
    """Scratch is kept per (device, stream): two calls of different shapes queued on two side
    streams at once give the same bits as the same calls on the default stream."""
    import torch

    import linear_complexity_vision_amd as L
    wa = workloads.make_random(201, 2, 1500, 130, dtype="bf16", w_range=5.0)
    wb = workloads.make_random(202, 1, 700, 64, dtype="f32", w_range=5.0)
    ga, gb = _upstream(wa, 203), _upstream(wb, 204)
    ta, tb = to_device_kv(wa), to_device_kv(wb)
    gda, gdb = torch.from_numpy(ga).cuda(), torch.from_numpy(gb).cuda()
    print("[case] backward on two side streams", flush=True)
    ref_a = [x.cpu().numpy() for x in L.biwkv_backward(*ta, gda)]
    ref_b = [x.cpu().numpy() for x in L.biwkv_backward(*tb, gdb)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        out_a = L.biwkv_backward(*ta, gda)
    with torch.cuda.stream(s2):
        out_b = L.biwkv_backward(*tb, gdb)
    torch.cuda.synchronize()
    for x, r in zip(out_a, ref_a):
        np.testing.assert_array_equal(x.cpu().numpy(), r)
    for x, r in zip(out_b, ref_b):
        np.testing.assert_array_equal(x.cpu().numpy(), r)


def _misaligned(t):
    """The same values at a 2-byte offset from a 4-byte boundary (a bf16 view one element into a
    larger buffer), so the bf16 channel-pair loads cannot be used."""
    import torch
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    m = flat[1:].view(t.shape)
    m.copy_(t)
    assert m.data_ptr() % 4 == 2
    return m


def test_backward_bf16_misaligned_even_channels():
    """Even C but k and v 2 bytes off a 4-byte boundary: the 16-bit loads instead of channel pairs,
    over several chunks per row, against the definition form."""
    import torch

    import linear_complexity_vision_amd as L
    wl = workloads.make_random(301, 2, 700, 66, dtype="bf16", w_range=6.0, k_std=1.5)
    gy = _upstream(wl, 302)
    k, v, w, u = to_device_kv(wl)
    print("[case] biwkv_backward bf16 misaligned k, v", flush=True)
    dk, dv, dw, du = L.biwkv_backward(_misaligned(k), _misaligned(v), w, u, torch.from_numpy(gy).cuda())
    torch.cuda.synchronize()
    got = (dk.cpu().numpy(), dv.cpu().numpy(), dw.cpu().numpy(), du.cpu().numpy())
    ref = oracle.biwkv_backward_sum(f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u), f64(gy), with_scale=True)
    for name, x, r, s in zip(("dk", "dv", "dw", "du"), got, ref[:4], ref[4:]):
        err = _scaled_err(x, r, s)
        print(f"[parity] backward misaligned {name}: scaled error {err:.3e}", flush=True)
        assert err <= 1e-4, (name, err)
    # the same bits as the aligned call (which takes the channel-pair loads)
    aligned = L.biwkv_backward(k, v, w, u, torch.from_numpy(gy).cuda())
    for x, a in zip(got, aligned):
        np.testing.assert_array_equal(x, a.cpu().numpy())
