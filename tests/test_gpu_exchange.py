"""GPU parity of the ways a row of several chunks is combined, and of the addressing limits.

* The two-pass form (chunk totals, per-chunk carries, then outputs; OPT_TWO_PASS = 1, which also
  applies to rows of one chunk) against the oracle, and bitwise reproducible.
* The one-launch exchange through each XCD's L2 (OPT_XCD_LOCAL = 1, the default) against the plain
  block order, bit for bit.
* The one-launch exchange with a poll limit of 0 (OPT_SPIN_LIMIT = 0): every workgroup recomputes
  every peer chunk's sums from k and v (the slow path taken when a peer is not resident), for
  every entry point built on the tile kernel; the fault word then reports the slow path.
* A batch item larger than 2 GiB of output (32-bit offsets only span one chunk).
* The 64-bit index form of the Q-Shift gathers: forced on small shapes, and reached naturally
  with more than 2^31 16-byte items.
* Scratch release, and backward calls from two host threads on one stream.

Bar as for the other parity tests: R3 <= 1e-4 (bf16 values are exact in the oracle); Q-Shift
bit for bit.
"""
import threading

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


def _entry(L, name, wl, k, v, w, u, r=None):
    if name == "biwkv":
        return L.biwkv_forward(k, v, w, u)
    if name == "fused":
        return L.biwkv_qshift_forward(k, v, w, u, wl.H, wl.W, wl.shift, wl.gamma)
    if name == "causal":
        return L.biwkv_causal_forward(k, v, w, u)
    if name == "gated":
        return L.biwkv_gated_forward(k, v, r, w, u)
    if name == "bidir":
        return L.biwkv_qshift_bidir_forward(k, v, w, u, wl.shift, wl.gamma)
    raise ValueError(name)


def _gate(wl):
    g = np.random.Generator(np.random.PCG64(77))
    r = (g.standard_normal(wl.k.shape) * 3.0).astype(np.float32)
    return workloads._to_bf16_values(r) if wl.dtype == "bf16" else r


def _oracle(name, wl, r=None):
    k, v, w, u = f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u)
    if name == "biwkv":
        return oracle.biwkv_rnn(k, v, w, u, with_scale=True)
    if name == "fused":
        return oracle.biwkv_qshift(k, v, w, u, wl.H, wl.W, wl.shift, wl.gamma, use_rnn=True, with_scale=True)
    if name == "causal":
        return oracle.biwkv_causal_rnn(k, v, w, u, with_scale=True)
    if name == "gated":
        return oracle.biwkv_gated(k, v, f64(r), w, u, with_scale=True)
    if name == "bidir":
        ks = oracle.qshift_bidir_f64(k, wl.shift, wl.gamma)
        vs = oracle.qshift_bidir_f64(v, wl.shift, wl.gamma)
        return oracle.biwkv_rnn(ks, vs, w, u, with_scale=True)
    raise ValueError(name)


def _device_gate(wl, r):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(workloads.round_to_bf16_bits(r))).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(r)).cuda()


def _run(name, wl, r=None):
    import torch
    L = _lib()
    k, v, w, u = to_device_kv(wl)
    rd = _device_gate(wl, r) if r is not None else None
    y = _entry(L, name, wl, k, v, w, u, rd)
    torch.cuda.synchronize()
    return y.cpu().numpy(), L.stream_fault_flags()


def _tol(wl):
    return 1e-4  # the wide form's exact token counts hold the plain bar for any w


# (entry, B, H, W, C, dtype): several chunks per row, ragged last chunk or tile where possible
MULTI_CHUNK = [
    ("biwkv", 1, 1, 1025, 64, "f32"), ("biwkv", 2, 1, 2047, 66, "bf16"), ("biwkv", 1, 1, 3000, 130, "f32"),
    ("biwkv", 1, 1, 5121, 32, "bf16"), ("biwkv", 2, 1, 1500, 3, "bf16"),
    ("fused", 1, 40, 50, 128, "bf16"), ("fused", 2, 33, 31, 66, "f32"),
    ("causal", 1, 1, 3000, 130, "bf16"), ("causal", 2, 1, 2047, 66, "f32"),
    ("gated", 1, 1, 2500, 130, "bf16"), ("gated", 1, 1, 1025, 64, "f32"),
    ("bidir", 2, 1, 2100, 96, "bf16"), ("bidir", 1, 1, 1300, 64, "f32"),
]


def _make(name, B, H, W, C, dtype, seed, w_range=6.0):
    wl = workloads.make_random(seed, B, H * W, C, dtype=dtype, w_range=w_range, k_std=2.0, u_std=1.5, H=H, W=W)
    wl.shift, wl.gamma = (2 if name == "bidir" else 1), 0.25
    return wl


@pytest.mark.parametrize("name,B,H,W,C,dtype", MULTI_CHUNK)
def test_two_pass_matches_oracle(name, B, H, W, C, dtype):
    L = _lib()
    wl = _make(name, B, H, W, C, dtype, seed=300 + H * W + C)
    r = _gate(wl) if name == "gated" else None
    print(f"[case] two passes {name} {wl.name}", flush=True)
    with L.option(L.OPT_TWO_PASS, 1):
        y2, f2 = _run(name, wl, r)
        y3, _ = _run(name, wl, r)
    assert f2 == 0
    np.testing.assert_array_equal(y2, y3)
    y_ref, s_ref = _oracle(name, wl, r)
    err = r3(y2, y_ref, s_ref)
    print(f"[parity] two passes {name} {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


# rows of one chunk in one launch (T <= 1024 for bf16, <= 512 for fp32) through the two-pass form
SINGLE_CHUNK = [("biwkv", 2, 1, 300, 100, "f32"), ("biwkv", 3, 1, 784, 130, "bf16"), ("fused", 4, 14, 14, 96, "f32"),
                ("causal", 2, 1, 700, 66, "bf16"), ("gated", 1, 1, 500, 64, "f32"), ("bidir", 2, 1, 49, 64, "f32"),
                ("biwkv", 1, 1, 1, 8, "f32"), ("biwkv", 2, 1, 129, 3, "bf16")]


@pytest.mark.parametrize("name,B,H,W,C,dtype", SINGLE_CHUNK)
def test_two_pass_single_chunk_rows(name, B, H, W, C, dtype):
    L = _lib()
    wl = _make(name, B, H, W, C, dtype, seed=350 + H * W + C)
    r = _gate(wl) if name == "gated" else None
    print(f"[case] two passes, short rows {name} {wl.name}", flush=True)
    with L.option(L.OPT_TWO_PASS, 1):
        y, _ = _run(name, wl, r)
    y_ref, s_ref = _oracle(name, wl, r)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] two passes, short rows {name} {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


@pytest.mark.parametrize("name,B,H,W,C,dtype", MULTI_CHUNK)
def test_recompute_every_peer(name, B, H, W, C, dtype):
    """A poll limit of 0: no workgroup waits, every peer chunk's sums come from k and v."""
    L = _lib()
    wl = _make(name, B, H, W, C, dtype, seed=400 + H * W + C)
    r = _gate(wl) if name == "gated" else None
    print(f"[case] recompute {name} {wl.name}", flush=True)
    with L.option(L.OPT_SPIN_LIMIT, 0):
        y, flags = _run(name, wl, r)
    assert flags & 1, "the slow path should be reported"
    y_ref, s_ref = _oracle(name, wl, r)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] recompute {name} {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


# rows of several chunks, 11 and 30 of them: the first 8 and 24 run each row on one XCD and
# exchange through its L2, the rest keep the plain order
XCD_ROWS = [("biwkv", 1, 1, 2500, 704, "f32"), ("fused", 3, 50, 60, 640, "bf16"), ("causal", 3, 1, 3000, 640, "bf16"),
            ("gated", 1, 1, 2100, 704, "f32"), ("bidir", 3, 1, 2100, 640, "bf16")]


@pytest.mark.parametrize("name,B,H,W,C,dtype", XCD_ROWS)
def test_xcd_local_exchange_matches_plain_order(name, B, H, W, C, dtype):
    """The one-launch exchange through each XCD's L2 gives the same bits as the plain block order
    (the fold order is fixed), and both match the oracle."""
    L = _lib()
    wl = _make(name, B, H, W, C, dtype, seed=500 + H * W + C)
    r = _gate(wl) if name == "gated" else None
    print(f"[case] XCD-local exchange {name} {wl.name}", flush=True)
    with L.option(L.OPT_XCD_LOCAL, 1):
        y1, f1 = _run(name, wl, r)
    with L.option(L.OPT_XCD_LOCAL, 0):
        y0, f0 = _run(name, wl, r)
    assert f1 == 0 and f0 == 0
    np.testing.assert_array_equal(y1, y0)
    y_ref, s_ref = _oracle(name, wl, r)
    err = r3(y1, y_ref, s_ref)
    print(f"[parity] XCD-local exchange {name} {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


@pytest.mark.parametrize("name,dtype", [("biwkv", "f32"), ("biwkv", "bf16"), ("causal", "f32"), ("gated", "f32")])
def test_one_launch_over_several_residency_rounds(name, dtype):
    """More workgroups than fit at once, with rows of 18 chunks: later rows start as earlier ones
    finish, and a row straddles the first round's end. No wait runs out (the fault word stays 0)
    and the outputs match the oracle; OPT_TWO_PASS = 2 and the default agree bit for bit."""
    L = _lib()
    T = 9000 if dtype == "f32" else 18000
    wl = _make(name, 2, 1, T, 1024, dtype, seed=600 + T)
    r = _gate(wl) if name == "gated" else None
    print(f"[case] one launch over several rounds {name} {wl.name}", flush=True)
    y, flags = _run(name, wl, r)
    with L.option(L.OPT_TWO_PASS, 2):
        y2, flags2 = _run(name, wl, r)
    assert flags == 0 and flags2 == 0
    np.testing.assert_array_equal(y, y2)
    y_ref, s_ref = _oracle(name, wl, r)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] one launch over several rounds {name} {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


def test_rows_longer_than_one_xcd_holds_keep_the_plain_order():
    """Rows of 40 chunks in 1024-thread workgroups: they fit the device at once (one launch over
    several rounds) but not one XCD's share of it, so they keep the plain block order. No wait may
    run out (the fault word stays 0), and the outputs match the oracle."""
    L = _lib()
    wl = _make("biwkv", 1, 1, 20480, 1024, "f32", seed=640)
    print(f"[case] rows of 40 chunks, one launch {wl.name}", flush=True)
    y, flags = _run("biwkv", wl)
    assert flags == 0
    y_ref, s_ref = _oracle("biwkv", wl)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] rows of 40 chunks: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_two_pass_rows_beyond_512_chunks(dtype):
    """A row of more than 64 * 8 chunks of 128 tokens: the carry kernel reads its totals from
    memory as it goes instead of holding them in registers."""
    L = _lib()
    wl = workloads.make_random(77, 1, 70001, 64, dtype=dtype, w_range=8.0, k_std=2.0)
    print(f"[case] two passes, 547 chunks per row {dtype}", flush=True)
    with L.option(L.OPT_TWO_PASS, 1):
        y, _ = _run("biwkv", wl)
    y_ref, s_ref = _oracle("biwkv", wl)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] two passes, 547 chunks per row {dtype}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4


@pytest.mark.parametrize("mode", ["two_pass", "recompute"])
@pytest.mark.parametrize("case", ["w_plus_1e4", "w_minus_1e4", "u_100", "k_plus_100"])
def test_wide_form_multi_chunk(mode, case):
    """The wide form (extreme w, u) of several chunks per row through both slow paths."""
    L = _lib()
    wl = workloads.make_random(55, 1, 2500, 64, dtype="f32", w_range=5.0)
    if case == "w_plus_1e4":
        wl.w[:] = 1e4
    elif case == "w_minus_1e4":
        wl.w[:] = -1e4
    elif case == "u_100":
        wl.u[:] = 100.0
    else:
        wl.k += np.float32(100.0)
    opt = (L.OPT_TWO_PASS, 1) if mode == "two_pass" else (L.OPT_SPIN_LIMIT, 0)
    print(f"[case] wide form {case} {mode}", flush=True)
    with L.option(*opt):
        y, _ = _run("biwkv", wl)
    y_ref, s_ref = oracle.biwkv_sum(f64(wl.k), f64(wl.v), f64(wl.w), f64(wl.u), with_scale=True)
    err = r3(y, y_ref, s_ref)
    tol = _tol(wl)
    print(f"[parity] wide form {case} {mode}: R3 = {err:.3e} (tol {tol:.1e})", flush=True)
    assert err <= tol


@pytest.mark.parametrize("index,fused", [(4, False), (4, True), (5, False)])
def test_workloads_through_slow_paths(index, fused):
    """The headline and stress workloads with every peer's sums recomputed (config 5 runs two
    launches by itself: its workgroups do not all fit at once)."""
    L = _lib()
    wl = workloads.make(index)
    name = "fused" if fused else "biwkv"
    print(f"[case] recompute {name} {wl.name}", flush=True)
    with L.option(L.OPT_SPIN_LIMIT, 0):
        y, _ = _run(name, wl)
    y_ref, s_ref = _oracle(name, wl)
    err = r3(y, y_ref, s_ref)
    print(f"[parity] recompute {name} {wl.name}: R3 = {err:.3e}", flush=True)
    assert err <= 1e-4
    if index == 4:
        with L.option(L.OPT_TWO_PASS, 1):
            y2, f2 = _run(name, wl)
        assert f2 == 0
        err2 = r3(y2, y_ref, s_ref)
        print(f"[parity] two passes {name} {wl.name}: R3 = {err2:.3e}", flush=True)
        assert err2 <= 1e-4


def _large_kv(seed, B, T, C):
    """Seeded N(0, 1) k and v of a large shape: float32 draws (generated in slices), rounded to
    bf16 by torch on the host (round to nearest even); returns host bf16 tensors."""
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(2):
        t = torch.empty((B, T, C), dtype=torch.bfloat16)
        for b in range(B):
            for t0 in range(0, T, 512):
                t1 = min(T, t0 + 512)
                t[b, t0:t1] = torch.from_numpy(rng.standard_normal((t1 - t0, C), dtype=np.float32)).to(torch.bfloat16)
        out.append(t)
    return out


@pytest.mark.parametrize("fused", [False, True])
def test_batch_item_beyond_2gib(fused):
    """One batch item of out spans more than 2^31 bytes (T = 4096, C = 131136): every chunk's
    resources start at the chunk, so 32-bit offsets still reach everything. Sampled channels
    (both ends, the Q-Shift group bounds, the middle) against the oracle."""
    import torch
    L = _lib()
    B, H, W, C = 1, 64, 64, 131136
    T = H * W
    print(f"[case] batch item beyond 2 GiB fused={fused}", flush=True)
    kh, vh = _large_kv(901, B, T, C)
    rng = np.random.Generator(np.random.PCG64(902))
    w = rng.uniform(-5, 5, C).astype(np.float32)
    u = rng.standard_normal(C).astype(np.float32)
    k, v = kh.cuda(), vh.cuda()
    wd, ud = torch.from_numpy(w).cuda(), torch.from_numpy(u).cuda()
    if fused:
        y = L.biwkv_qshift_forward(k, v, wd, ud, H, W, 1, 0.25)
    else:
        y = L.biwkv_forward(k, v, wd, ud)
    torch.cuda.synchronize()
    g = [int(C * 0.25 * j) for j in (1, 2, 3, 4)]
    sel = sorted(set(list(range(0, 8)) + list(range(C - 8, C)) + [C // 2, C // 2 + 1]
                     + [x + d for x in g for d in (-1, 0) if 0 <= x + d < C]))
    sel = np.array(sel)
    ys = y[:, :, torch.from_numpy(sel).cuda()].cpu().numpy()
    del y, k, v
    torch.cuda.empty_cache()
    kf = kh.float().numpy()
    vf = vh.float().numpy()
    if fused:
        # the oracle's gather on the whole item (bit copies in float32), then the sampled channels
        ks = oracle.qshift(kf, H, W, 1, 0.25)[:, :, sel]
        vs = oracle.qshift(vf, H, W, 1, 0.25)[:, :, sel]
    else:
        ks, vs = kf[:, :, sel], vf[:, :, sel]
    y_ref, s_ref = oracle.biwkv_rnn(f64(ks), f64(vs), f64(w[sel]), f64(u[sel]), with_scale=True)
    err = r3(ys, y_ref, s_ref)
    print(f"[parity] beyond 2 GiB fused={fused}: R3 = {err:.3e} on {sel.size} channels", flush=True)
    assert err <= 1e-4


@pytest.mark.parametrize("B,H,W,C,shift,gamma", [
    (3, 37, 41, 1000, 2, 0.25), (2, 14, 14, 384, 1, 0.25), (1, 5, 7, 100, 2, 0.125), (2, 6, 2, 10, 2, 0.2)])
def test_wide_index_gathers_bit_exact(B, H, W, C, shift, gamma):
    """The 64-bit index form of the Q-Shift gather, the mixing kernel and the sequence shift,
    forced on small shapes, bit for bit against the oracle."""
    import torch
    L = _lib()
    g = np.random.Generator(np.random.PCG64(B * 7 + H * W + C))
    bits = g.integers(0, 2**32, size=(B, H * W, C), dtype=np.uint64).astype(np.uint32)
    bits.reshape(-1)[:4] = [0x7FC00001, 0xFF800000, 0x80000000, 0x00000003]
    x = torch.from_numpy(bits.view(np.float32)).cuda()
    mu = torch.from_numpy(g.uniform(0, 1, (3, C)).astype(np.float32)).cuda()
    xv = torch.from_numpy(g.standard_normal((B, H * W, C)).astype(np.float32)).cuda()  # mixing inputs
    print(f"[case] 64-bit index gathers B{B} H{H} W{W} C{C}", flush=True)
    with L.option(L.OPT_WIDE_INDEX, 1):
        q = L.qshift(x, H, W, shift, gamma).cpu().numpy()
        qb = L.qshift_bidir(x, shift, gamma).cpu().numpy()
        m = L.qshift_mix(xv, mu, H, W, shift, gamma).cpu().numpy()
    np.testing.assert_array_equal(q.view(np.uint32), oracle.qshift(bits.view(np.float32), H, W, shift, gamma).view(np.uint32))
    np.testing.assert_array_equal(qb.view(np.uint32), oracle.qshift_bidir(bits.view(np.float32), shift, gamma).view(np.uint32))
    with L.option(L.OPT_WIDE_INDEX, 0):
        m32 = L.qshift_mix(xv, mu, H, W, shift, gamma).cpu().numpy()
    np.testing.assert_array_equal(m, m32)
    # Eq. (9) in fp32: within two roundings of the terms' magnitudes of the float64 oracle
    xh, muh = xv.cpu().numpy(), mu.cpu().numpy()
    ref = oracle.qshift_mix(xh, muh, H, W, shift, gamma)
    xd = oracle.qshift_f64(xh, H, W, shift, gamma)
    bound = 2.0 * 2.0 ** -23 * (np.abs(f64(xh))[None] + np.abs((1.0 - f64(muh))[:, None, None, :] * xd[None]))
    assert not (np.abs(f64(m) - ref) > bound).any()


def test_qshift_beyond_2_31_items():
    """More than 2^31 16-byte items (B = 2100 of 64 x 64 x 1024 fp32, 35 GB in and out): the
    gather takes its 64-bit index form by itself. The input is a fixed bit pattern per batch item
    (x[b] = base ^ b, NaN payloads included); the items on both sides of index 2^31 and the last
    ones are compared bit for bit with the oracle."""
    import torch
    L = _lib()
    B, H, W, C = 2100, 64, 64, 1024
    assert B * H * W * C // 4 >= 2**31
    print("[case] qshift beyond 2^31 items (70 GB on the device)", flush=True)
    g = np.random.Generator(np.random.PCG64(2100))
    base = g.integers(0, 2**32, size=(H * W, C), dtype=np.uint64).astype(np.uint32)
    base[0, :4] = [0x7FC00001, 0xFF800000, 0x80000000, 0x00000003]
    base_d = torch.from_numpy(base.view(np.int32)).cuda()
    x = torch.empty((B, H * W, C), dtype=torch.int32, device="cuda")
    for b in range(B):
        torch.bitwise_xor(base_d, b, out=x[b])
    out = L.qshift(x.view(torch.float32), H, W, 1, 0.25)
    torch.cuda.synchronize()
    for b in (0, 2047, 2048, 2049, B - 1):
        xb = (base ^ np.uint32(b)).reshape(1, H * W, C)
        ref = oracle.qshift(xb.view(np.float32), H, W, 1, 0.25).view(np.uint32)
        np.testing.assert_array_equal(out[b:b + 1].cpu().numpy().view(np.uint32), ref)
    del x, out
    torch.cuda.empty_cache()


def test_release_scratch_then_reuse():
    import torch
    L = _lib()
    wl = workloads.make_random(31, 2, 3000, 128, dtype="bf16")
    k, v, w, u = to_device_kv(wl)
    s = torch.cuda.Stream()
    print("[case] release scratch", flush=True)
    with torch.cuda.stream(s):
        a = L.biwkv_forward(k, v, w, u)
        L.release_scratch()
        L.release_scratch()  # nothing left: still fine
        b = L.biwkv_forward(k, v, w, u)  # fresh scratch on the same stream
        c = L.biwkv_forward(k, v, w, u)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    np.testing.assert_array_equal(a.cpu().numpy(), c.cpu().numpy())
    with torch.cuda.stream(s):
        assert L.stream_fault_flags() == 0
        L.release_scratch()
    torch.cuda.synchronize()


def test_backward_from_two_threads_on_one_stream():
    """Two host threads call the backward (six launches sharing the stream's scratch) on the same
    stream with different inputs: each result equals its single-threaded one bit for bit."""
    import torch
    L = _lib()
    wls = [workloads.make_random(61 + i, 2, 4096, 128, dtype="bf16") for i in range(2)]
    devs = [to_device_kv(wl) for wl in wls]
    gys = [torch.from_numpy(np.random.Generator(np.random.PCG64(71 + i)).standard_normal(
        wls[i].k.shape).astype(np.float32)).cuda() for i in range(2)]
    print("[case] backward from two threads", flush=True)
    ref = []
    for i in range(2):
        k, v, w, u = devs[i]
        ref.append([t.cpu().numpy() for t in L.biwkv_backward(k, v, w, u, gys[i])])
    torch.cuda.synchronize()
    results = [[], []]
    stream = torch.cuda.current_stream()

    def worker(i):
        with torch.cuda.stream(stream):
            k, v, w, u = devs[i]
            for _ in range(6):
                results[i].append(L.biwkv_backward(k, v, w, u, gys[i]))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i in range(2):
        for res in results[i]:
            for got, want in zip(res, ref[i]):
                np.testing.assert_array_equal(got.cpu().numpy(), want)
