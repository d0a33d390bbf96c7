"""GPU parity of the bidirectional shift for sparse (MAE-masked) inputs, through the C ABI:
qshift_bidir bit for bit against the oracle's gather, and the fused biwkv_qshift_bidir_forward
against the float64 oracle (Bi-WKV of the oracle-shifted k and v; Eq. (5) of the Vision-RWKV
article, section "MAE pre-training" for the shift). Bar: R3 <= 1e-4 (bf16 values are exact in the
oracle); extreme-w cases use the fp32 exponent-resolution bound of the forward tests.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import f64, to_device_kv
from tests.metrics import r3

pytestmark = pytest.mark.gpu


def _lib():
    import linear_complexity_vision_amd as L
    return L


def _fused(wl, shift, gamma):
    import torch
    L = _lib()
    k, v, w, u = to_device_kv(wl)
    y = L.biwkv_qshift_bidir_forward(k, v, w, u, shift, gamma)
    torch.cuda.synchronize()
    assert L.stream_fault_flags() == 0
    return y.cpu().numpy()


def _ref(wl, shift, gamma, use_sum):
    ks = oracle.qshift_bidir_f64(f64(wl.k), shift, gamma)
    vs = oracle.qshift_bidir_f64(f64(wl.v), shift, gamma)
    fn = oracle.biwkv_sum if use_sum else oracle.biwkv_rnn
    return fn(ks, vs, f64(wl.w), f64(wl.u), with_scale=True)


@pytest.mark.parametrize("index", sorted(workloads.MAE_SPECS))
def test_bidir_gather_workloads_bit_exact(index):
    import torch
    wl = workloads.make_mae(index)
    print(f"[case] qshift_bidir {wl.name}", flush=True)
    out = _lib().qshift_bidir(torch.from_numpy(wl.k).cuda(), 1, 0.25).cpu().numpy()
    np.testing.assert_array_equal(out.view(np.uint32), oracle.qshift_bidir(wl.k, 1, 0.25).view(np.uint32))


@pytest.mark.parametrize("B,N,C,shift,gamma", [
    (2, 49, 384, 1, 0.25), (1, 35, 100, 2, 0.125), (3, 16, 17, 3, 0.25), (2, 12, 10, 2, 0.2),
    (1, 1, 8, 1, 0.25), (1, 9, 12, 0, 0.25), (1, 9, 12, 1, 0.0), (2, 16, 8, 16, 0.25), (1, 1000, 64, 5, 0.25)])
def test_bidir_gather_bit_patterns(B, N, C, shift, gamma):
    """Random 32-bit patterns, NaN payloads, -0.0 and denormals move unchanged."""
    import torch
    print(f"[case] qshift_bidir B{B} N{N} C{C} s{shift} g{gamma}", flush=True)
    g = np.random.Generator(np.random.PCG64(B * 1000 + N * 10 + C))
    bits = g.integers(0, 2**32, size=(B, N, C), dtype=np.uint64).astype(np.uint32)
    special = np.array([0x7FC00001, 0xFF800000, 0x80000000, 0x00000003], dtype=np.uint32)
    bits.reshape(-1)[: special.size] = special[: bits.size]
    out = _lib().qshift_bidir(torch.from_numpy(bits.view(np.float32)).cuda(), shift, gamma)
    ref = oracle.qshift_bidir(bits.view(np.float32), shift, gamma).view(np.uint32)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref)


@pytest.mark.parametrize("index", sorted(workloads.MAE_SPECS))
def test_fused_bidir_workloads(index):
    wl = workloads.make_mae(index)
    print(f"[case] biwkv_qshift_bidir_forward {wl.name}", flush=True)
    y = _fused(wl, 1, 0.25)
    assert np.isfinite(y).all()
    y_ref, s_ref = _ref(wl, 1, 0.25, use_sum=False)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] fused bidir {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


BIDIR_SHAPES = [(1, 1, 4, 1, 0.25), (2, 2, 6, 1, 0.25), (1, 3, 8, 3, 0.25), (1, 129, 66, 1, 0.25),
                (2, 255, 130, 2, 0.2), (1, 513, 64, 1, 0.125), (3, 200, 100, 1, 0.25), (1, 700, 10, 4, 0.2),
                # several chunks per row, ragged last chunk and tile, shifts across chunk seams
                (1, 1025, 64, 1, 0.25), (2, 2047, 66, 3, 0.25), (1, 3000, 130, 1, 0.25), (1, 5121, 32, 2, 0.25),
                (1, 600, 16, 600, 0.25)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,N,C,shift,gamma", BIDIR_SHAPES)
def test_fused_bidir_edge_shapes(B, N, C, shift, gamma, dtype):
    wl = workloads.make_random(300 + N + C + shift, B, N, C, dtype=dtype, w_range=6.0, k_std=2.0)
    print(f"[case] biwkv_qshift_bidir_forward edge {wl.name} s{shift} g{gamma}", flush=True)
    y = _fused(wl, shift, gamma)
    y_ref, s_ref = _ref(wl, shift, gamma, use_sum=True)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] fused bidir edge {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


def test_fused_bidir_equals_gather_then_biwkv():
    """fp32: the fused loads and the standalone gather feed the tile kernel the same values, so
    the outputs agree bit for bit; ten fused runs are identical."""
    import torch
    L = _lib()
    wl = workloads.make_random(77, 2, 3000, 128, dtype="f32", w_range=5.0)
    k, v, w, u = to_device_kv(wl)
    print("[case] fused bidir vs gather + biwkv_forward, determinism", flush=True)
    yf = L.biwkv_qshift_bidir_forward(k, v, w, u, 2, 0.25)
    yu = L.biwkv_forward(L.qshift_bidir(k, 2, 0.25), L.qshift_bidir(v, 2, 0.25), w, u)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(yf.cpu().numpy(), yu.cpu().numpy())
    first = yf.cpu().numpy()
    for _ in range(10):
        np.testing.assert_array_equal(L.biwkv_qshift_bidir_forward(k, v, w, u, 2, 0.25).cpu().numpy(), first)
    assert L.stream_fault_flags() == 0


@pytest.mark.parametrize("case", ["k_plus_100", "w_plus_1e4", "w_minus_1e4"])
def test_fused_bidir_extreme_values(case):
    wl = workloads.make_random(99, 1, 2500, 64, dtype="f32", w_range=5.0)
    if case == "k_plus_100":
        wl.k = wl.k + np.float32(100.0)
    elif case == "w_plus_1e4":
        wl.w = np.full_like(wl.w, 1e4)
    else:
        wl.w = np.full_like(wl.w, -1e4)
    print(f"[case] biwkv_qshift_bidir_forward extreme {case}", flush=True)
    y = _fused(wl, 1, 0.25)
    assert np.isfinite(y).all()
    y_ref, s_ref = _ref(wl, 1, 0.25, use_sum=True)
    tol = 1e-4  # the wide form's exact token counts hold the plain bar at |w| = 1e4
    err = r3(y, y_ref, s_ref)
    print(f"[parity] fused bidir extreme {case}: R3 = {err:.3e} (tol {tol:.1e})", flush=True)
    assert err <= tol
