"""GPU parity on seeded random shapes, entries and launch options, through the C ABI: every
forward entry (plain, fused Q-Shift, causal, gated, sparse bidirectional shift) on shapes drawn
across the tile kernel's shape boundaries (one chunk or several; rows fewer or more than the CUs;
ragged last tile and chunk) and under each combination of the exchange options (rows on one XCD
or in plain order; one launch, two passes, or one launch whenever a row fits). Outputs are
compared with the float64 RNN-form oracle (R3 <= 1e-4, Eq. (5) of the Vision-RWKV article), and a
launch must never report a wait that ran out.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import f64, to_device_kv
from tests.metrics import r3

pytestmark = pytest.mark.gpu

ENTRIES = ("biwkv", "fused", "causal", "gated", "bidir")


def _case(i):
    """Case i: (entry, B, H, W, C, dtype, two_pass option, xcd option), from its own seed."""
    g = np.random.Generator(np.random.PCG64(7000 + i))
    entry = ENTRIES[i % len(ENTRIES)]
    dtype = "bf16" if g.random() < 0.5 else "f32"
    if g.random() < 0.35:
        # many rows (more than one round of one workgroup per CU), short rows
        T = int(g.integers(1, 1100))
        C = int(g.integers(3000, 4200))
        B = int(g.integers(4, 6))
    else:
        T = int(g.integers(1, 9000))
        C = int(g.integers(1, 700))
        B = int(g.integers(1, 4))
    if entry == "fused":
        W = int(g.integers(1, 80))
        H = max(1, T // W)
    else:
        H, W = 1, T
    two_pass = int(g.integers(0, 3))
    xcd = int(g.integers(0, 2))
    return entry, B, H, W, C, dtype, two_pass, xcd


CASES = [_case(i) for i in range(40)]


@pytest.mark.parametrize("entry,B,H,W,C,dtype,two_pass,xcd", CASES)
def test_random_shape(entry, B, H, W, C, dtype, two_pass, xcd):
    import torch

    import linear_complexity_vision_amd as L
    T = H * W
    wl = workloads.make_random(8000 + B * 7 + T + C, B, T, C, dtype=dtype, w_range=6.0, k_std=2.0, u_std=1.5,
                               H=H, W=W)
    shift = 2 if entry == "bidir" else 1
    r = None
    if entry == "gated":
        gr = np.random.Generator(np.random.PCG64(T + C))
        r = (gr.standard_normal(wl.k.shape) * 3.0).astype(np.float32)
        if dtype == "bf16":
            r = workloads._to_bf16_values(r)
    print(f"[case] random {entry} {wl.name} H{H} W{W} two_pass={two_pass} xcd={xcd}", flush=True)
    k, v, w, u = to_device_kv(wl)
    with L.option(L.OPT_TWO_PASS, two_pass), L.option(L.OPT_XCD_LOCAL, xcd):
        if entry == "biwkv":
            y = L.biwkv_forward(k, v, w, u)
        elif entry == "fused":
            y = L.biwkv_qshift_forward(k, v, w, u, H, W, shift, 0.25)
        elif entry == "causal":
            y = L.biwkv_causal_forward(k, v, w, u)
        elif entry == "gated":
            if dtype == "bf16":
                rd = torch.from_numpy(np.ascontiguousarray(workloads.round_to_bf16_bits(r))).view(torch.bfloat16).cuda()
            else:
                rd = torch.from_numpy(np.ascontiguousarray(r)).cuda()
            y = L.biwkv_gated_forward(k, v, rd, w, u)
        else:
            y = L.biwkv_qshift_bidir_forward(k, v, w, u, shift, 0.25)
        torch.cuda.synchronize()
        flags = L.stream_fault_flags()
    y = y.cpu().numpy()
    kk, vv, ww, uu = f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u)
    if entry == "biwkv":
        y_ref, s_ref = oracle.biwkv_rnn(kk, vv, ww, uu, with_scale=True)
    elif entry == "fused":
        y_ref, s_ref = oracle.biwkv_qshift(kk, vv, ww, uu, H, W, shift, 0.25, use_rnn=True, with_scale=True)
    elif entry == "causal":
        y_ref, s_ref = oracle.biwkv_causal_rnn(kk, vv, ww, uu, with_scale=True)
    elif entry == "gated":
        y_ref, s_ref = oracle.biwkv_gated(kk, vv, f64(r), ww, uu, with_scale=True)
    else:
        ks = oracle.qshift_bidir_f64(kk, shift, 0.25)
        vs = oracle.qshift_bidir_f64(vv, shift, 0.25)
        y_ref, s_ref = oracle.biwkv_rnn(ks, vs, ww, uu, with_scale=True)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] random {entry} {wl.name}: R3 = {err:.3e}", flush=True)
    assert flags == 0, "a wait ran out"
    assert err <= 1e-4
