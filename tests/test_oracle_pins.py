"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

The oracle computes Bi-WKV (Eq. (5)-(7) of the Vision-RWKV article, section "Linear Complexity
Bidirectional Attention") and Q-Shift (the q_shift function of LinXin's Blog notes). Nothing here
re-types the oracle's formula: each test is a hand-derived fixture, a closed form or limit, an
invariant of Eq. (5), agreement between two different evaluation orders written independently,
or a brute-force gather formulated differently (np.roll + masks).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from tests.metrics import r3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LN2 = float(np.log(2.0))


def _rng(seed):
    return np.random.Generator(np.random.PCG64(1000 + seed))


def _rand(seed, B, T, C, kstd=1.0, wr=5.0, ustd=1.0):
    g = _rng(seed)
    k = g.standard_normal((B, T, C)) * kstd
    v = g.standard_normal((B, T, C))
    w = g.uniform(-wr, wr, C)
    u = g.standard_normal(C) * ustd
    return k, v, w, u


def _read_biwkv_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "biwkv_hand_T4.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0]}
                cases.append(cur)
            elif key == "y":
                cur["y"] = [float(Fraction(x)) for x in vals]
            elif key in ("k", "v"):
                cur[key] = [float(x) for x in vals]
            else:
                cur[key] = float(vals[0])
    return cases


@pytest.mark.parametrize("case", _read_biwkv_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("form", ["sum", "rnn", "literal"])
def test_hand_fixture(case, form):
    T = int(case["T"])
    k = np.array(case["k"]).reshape(1, T, 1)
    v = np.array(case["v"]).reshape(1, T, 1)
    w, u = np.array([case["w"]]), np.array([case["u"]])
    fn = {"sum": oracle.biwkv_sum, "rnn": oracle.biwkv_rnn, "literal": oracle.biwkv_rnn_literal}[form]
    y = fn(k, v, w, u).reshape(-1)
    np.testing.assert_allclose(y, case["y"], rtol=1e-14, atol=0)


def test_hand_fixture_as_channels():
    """All T = 4 cases side by side as channels of one call (per-channel w and u)."""
    cases = [c for c in _read_biwkv_cases() if int(c["T"]) == 4]
    k = np.stack([c["k"] for c in cases], axis=-1)[None]
    v = np.stack([c["v"] for c in cases], axis=-1)[None]
    w = np.array([c["w"] for c in cases])
    u = np.array([c["u"] for c in cases])
    y_ref = np.stack([c["y"] for c in cases], axis=-1)[None]
    for fn in (oracle.biwkv_sum, oracle.biwkv_rnn):
        np.testing.assert_allclose(fn(k, v, w, u), y_ref, rtol=1e-14, atol=0)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8, 17, 64])
@pytest.mark.parametrize("C", [1, 3, 8])
@pytest.mark.parametrize("B", [1, 2])
def test_sum_equals_rnn(T, C, B):
    """The two forms of the article (Eq. (5) vs Eq. (6)-(7)) agree: summation vs recurrence."""
    k, v, w, u = _rand(T * 100 + C * 10 + B, B, T, C, kstd=4.0, wr=8.0)
    y1, s1 = oracle.biwkv_sum(k, v, w, u, with_scale=True)
    y2, s2 = oracle.biwkv_rnn(k, v, w, u, with_scale=True)
    assert r3(y2, y1, s1) <= 1e-12
    np.testing.assert_allclose(s2, s1, rtol=1e-12)


@pytest.mark.parametrize("T", [2, 5, 11, 32])
def test_literal_recurrence_equals_sum(T):
    k, v, w, u = _rand(T, 2, T, 4, kstd=1.0, wr=2.0)
    y1, s1 = oracle.biwkv_sum(k, v, w, u, with_scale=True)
    y3 = oracle.biwkv_rnn_literal(k, v, w, u)
    assert r3(y3, y1, s1) <= 1e-9


@pytest.mark.parametrize("T", [3, 16, 64])
def test_single_query_softmax_with_linear_bias(T):
    """Per channel, Eq. (5) is single-query softmax attention whose bias is linear in the token
    distance (an ALiBi-like term): scipy's softmax over logits built from |t - i| gives y."""
    k, v, w, u = _rand(T + 7, 1, T, 5, kstd=2.0, wr=6.0)
    dist = np.abs(np.subtract.outer(np.arange(T), np.arange(T))).astype(np.float64)
    y_ref = np.empty((1, T, 5))
    for c in range(5):
        logits = -(dist - 1.0) / T * w[c] + k[0, :, c][None, :]
        np.fill_diagonal(logits, u[c] + k[0, :, c])
        y_ref[0, :, c] = softmax(logits, axis=1) @ v[0, :, c]
    y1 = oracle.biwkv_sum(k, v, w, u)
    np.testing.assert_allclose(y1, y_ref, rtol=1e-12, atol=1e-13)


def test_T1_is_identity():
    k, v, w, u = _rand(1, 3, 1, 6, kstd=3.0)
    np.testing.assert_array_equal(oracle.biwkv_sum(k, v, w, u), v)
    for fn in (oracle.biwkv_rnn, oracle.biwkv_rnn_literal):
        np.testing.assert_allclose(fn(k, v, w, u), v, rtol=2.3e-16, atol=0)


def test_T2_independent_of_w():
    k, v, _, u = _rand(2, 2, 2, 4)
    ya = oracle.biwkv_sum(k, v, np.full(4, -50.0), u)
    yb = oracle.biwkv_sum(k, v, np.full(4, 123.0), u)
    ek = np.exp(k)
    eu = np.exp(u)
    y0 = (ek[:, 1] * v[:, 1] + eu * ek[:, 0] * v[:, 0]) / (ek[:, 1] + eu * ek[:, 0])
    y1 = (ek[:, 0] * v[:, 0] + eu * ek[:, 1] * v[:, 1]) / (ek[:, 0] + eu * ek[:, 1])
    np.testing.assert_allclose(ya[:, 0], y0, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ya[:, 1], y1, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(yb, ya)


@pytest.mark.parametrize("T", [3, 10, 50])
def test_constant_k_zero_decay_closed_form(T):
    """w = 0, constant k: y_t = (sum_{i != t} v_i + e^u v_t) / (T - 1 + e^u); u = 0 gives the mean."""
    g = _rng(T)
    C = 4
    v = g.standard_normal((1, T, C))
    k = np.full((1, T, C), 0.37)
    w = np.zeros(C)
    u = np.array([0.0, 1.0, -2.0, 3.5])
    eu = np.exp(u)
    tot = v.sum(axis=1, keepdims=True)
    y_ref = (tot - v + eu * v) / (T - 1 + eu)
    for fn in (oracle.biwkv_sum, oracle.biwkv_rnn):
        y = fn(k, v, w, u)
        np.testing.assert_allclose(y, y_ref, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(y[..., 0], np.broadcast_to(v.mean(axis=1)[:, None, 0], (1, T)), rtol=1e-13)


def test_large_bonus_gives_v():
    k, v, w, _ = _rand(5, 2, 20, 3)
    np.testing.assert_allclose(oracle.biwkv_sum(k, v, w, np.full(3, 700.0)), v, rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(oracle.biwkv_rnn(k, v, w, np.full(3, 600.0)), v, rtol=1e-15, atol=1e-300)


@pytest.mark.parametrize("T", [3, 9, 64])
def test_strong_decay_gives_three_tap(T):
    """w -> +inf: only distance-1 neighbours (no decay) and the self term survive; this pins the
    '-1' in |t-i|-1 and the division by T."""
    k, v, _, u = _rand(T + 3, 1, T, 3)
    w = np.full(3, 1e5)
    y = oracle.biwkv_sum(k, v, w, u)
    ek, eu = np.exp(k), np.exp(u)
    num = eu * ek * v
    den = eu * ek
    num[:, 1:] += ek[:, :-1] * v[:, :-1]
    den[:, 1:] += ek[:, :-1]
    num[:, :-1] += ek[:, 1:] * v[:, 1:]
    den[:, :-1] += ek[:, 1:]
    np.testing.assert_allclose(y, num / den, rtol=1e-12)


@pytest.mark.parametrize("T", [3, 4, 9, 30])
def test_strong_growth_gives_farthest_endpoint(T):
    """w -> -inf: the farthest token dominates (v_{T-1} left of centre, v_0 right of centre,
    their e^k-weighted mean at the centre of an odd-length sequence)."""
    k, v, _, u = _rand(T + 11, 1, T, 2)
    y = oracle.biwkv_sum(k, v, np.full(2, -1e5), u)
    for t in range(T):
        if 2 * t < T - 1:
            ref = v[0, T - 1]
        elif 2 * t > T - 1:
            ref = v[0, 0]
        elif T == 3:
            # both endpoints sit at distance 1 (no decay at all): plain 3-tap weighted mean
            e = np.exp(k[0]).copy()
            e[1] *= np.exp(u)
            ref = (e * v[0]).sum(axis=0) / e.sum(axis=0)
        else:
            e0, e1 = np.exp(k[0, 0]), np.exp(k[0, T - 1])
            ref = (e0 * v[0, 0] + e1 * v[0, T - 1]) / (e0 + e1)
        np.testing.assert_allclose(y[0, t], ref, rtol=1e-12)


def test_reversal_symmetry():
    k, v, w, u = _rand(21, 2, 37, 5, kstd=3.0, wr=8.0)
    y = oracle.biwkv_sum(k, v, w, u)
    yr = oracle.biwkv_sum(k[:, ::-1], v[:, ::-1], w, u)
    np.testing.assert_allclose(yr[:, ::-1], y, rtol=1e-13, atol=1e-14)
    yr2 = oracle.biwkv_rnn(k[:, ::-1], v[:, ::-1], w, u)
    np.testing.assert_allclose(yr2[:, ::-1], y, rtol=1e-12, atol=1e-13)


def test_affine_in_v():
    k, v, w, u = _rand(22, 1, 40, 4)
    y = oracle.biwkv_sum(k, v, w, u)
    np.testing.assert_allclose(oracle.biwkv_sum(k, 2.5 * v - 1.25, w, u), 2.5 * y - 1.25, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("shift", [-100.0, 100.0, 600.0, -600.0])
def test_invariant_to_per_channel_k_shift(shift):
    k, v, w, u = _rand(23, 1, 40, 4, kstd=2.0)
    y = oracle.biwkv_sum(k, v, w, u)
    kk = k + shift * np.array([1.0, -1.0, 0.5, 0.0])
    np.testing.assert_allclose(oracle.biwkv_sum(kk, v, w, u), y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.biwkv_rnn(kk, v, w, u), y, rtol=1e-12, atol=1e-13)


def test_convexity():
    k, v, w, u = _rand(24, 2, 60, 6, kstd=4.0, wr=8.0, ustd=3.0)
    y = oracle.biwkv_sum(k, v, w, u)
    lo = v.min(axis=1, keepdims=True)
    hi = v.max(axis=1, keepdims=True)
    eps = 1e-14
    assert np.all(y >= lo - eps) and np.all(y <= hi + eps)


def test_channel_permutation_and_batch_independence():
    k, v, w, u = _rand(25, 3, 19, 7, kstd=2.0)
    y = oracle.biwkv_sum(k, v, w, u)
    perm = _rng(99).permutation(7)
    np.testing.assert_array_equal(oracle.biwkv_sum(k[..., perm], v[..., perm], w[perm], u[perm]), y[..., perm])
    np.testing.assert_array_equal(oracle.biwkv_sum(k[1:2], v[1:2], w, u), y[1:2])


def test_row_subset_matches_full():
    k, v, w, u = _rand(26, 2, 33, 3)
    y, s = oracle.biwkv_sum(k, v, w, u, with_scale=True)
    rows = [0, 5, 17, 32]
    ys, ss = oracle.biwkv_sum(k, v, w, u, rows=rows, with_scale=True)
    np.testing.assert_array_equal(ys, y[:, rows])
    np.testing.assert_array_equal(ss, s[:, rows])


def test_scale_bounds_output():
    k, v, w, u = _rand(27, 1, 50, 4)
    y, s = oracle.biwkv_sum(k, v, w, u, with_scale=True)
    assert np.all(np.abs(y) <= s * (1 + 1e-14))
    np.testing.assert_allclose(oracle.biwkv_sum(k, np.abs(v), w, u), s, rtol=1e-14)


# --------------------------------------------------------------------------------------------
# Q-Shift pins
# --------------------------------------------------------------------------------------------

def _qshift_roll(x, H, W, shift, gamma):
    """Independent formulation: np.roll along the grid axes, then zero what wrapped around."""
    B, N, C = x.shape
    g = [int(C * gamma * j) for j in (1, 2, 3, 4)]
    grid = x.reshape(B, H, W, C)
    out = grid.copy()
    s = shift
    zero = np.zeros((), dtype=x.dtype)
    parts = [(0, g[0], 2, s), (g[0], g[1], 2, -s), (g[1], g[2], 1, s), (g[2], g[3], 1, -s)]
    for lo, hi, axis, sh in parts:
        if hi <= lo:
            continue
        rolled = np.roll(grid[..., lo:hi], sh, axis=axis)
        idx = np.arange(grid.shape[axis])
        bad = (idx < sh) if sh >= 0 else (idx >= grid.shape[axis] + sh)
        shape = [1, 1, 1, 1]
        shape[axis] = -1
        rolled = np.where(bad.reshape(shape), zero, rolled)
        out[..., lo:hi] = rolled
    return out.reshape(B, N, C)


def test_qshift_hand_fixture():
    meta, rows = {}, []
    with open(os.path.join(GOLDEN, "qshift_hand_H2_W3_C5.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0].isalpha():
                meta[parts[0]] = float(parts[1])
            else:
                rows.append([float(p) for p in parts])
    H, W, C = int(meta["H"]), int(meta["W"]), int(meta["C"])
    x = np.empty((1, H * W, C), dtype=np.float32)
    for h in range(H):
        for w in range(W):
            for c in range(C):
                x[0, h * W + w, c] = 1000 + 100 * c + 10 * h + w
    out = oracle.qshift(x, H, W, int(meta["shift"]), meta["gamma"])
    exp = np.array([r[1:] for r in rows], dtype=np.float32)[None]
    np.testing.assert_array_equal(out, exp)


@pytest.mark.parametrize("H,W,C,shift,gamma", [
    (14, 14, 384, 1, 0.25), (3, 4, 10, 1, 0.2), (5, 7, 100, 2, 0.125), (4, 4, 17, 3, 0.25),
    (6, 2, 9, 2, 0.25), (1, 8, 8, 1, 0.25), (8, 1, 8, 1, 0.1)])
def test_qshift_bitwise_against_roll_formulation(H, W, C, shift, gamma):
    g = _rng(H * 31 + W)
    bits = g.integers(0, 2**32, size=(2, H * W, C), dtype=np.uint64).astype(np.uint32)
    bits[0, 0, : min(C, 4)] = [0x7FC00000, 0x7F800001, 0x00000001, 0x80000000][: min(C, 4)]
    x = bits.view(np.float32)
    out = oracle.qshift(x, H, W, shift, gamma)
    ref = _qshift_roll(bits, H, W, shift, gamma)
    np.testing.assert_array_equal(out.view(np.uint32), ref)


@pytest.mark.parametrize("H,W,C,shift,gamma", [(14, 14, 384, 1, 0.25), (5, 7, 100, 2, 0.125), (9, 6, 13, 3, 0.2)])
def test_qshift_zero_count(H, W, C, shift, gamma):
    x = np.ones((2, H * W, C), dtype=np.float32)
    out = oracle.qshift(x, H, W, shift, gamma)
    g2, g4 = int(C * gamma * 2), int(C * gamma * 4)
    expect = shift * H * g2 + shift * W * (g4 - g2)
    assert int((out[0] == 0).sum()) == expect
    assert np.all(np.signbit(out[out == 0]) == 0)  # zero fill is +0.0


def test_qshift_boundaries_C100_gamma_eighth():
    """C = 100, gamma = 1/8: int(12.5) = 12, 25, int(37.5) = 37, 50; channels >= 50 copied."""
    H, W = 3, 3
    x = np.ones((1, 9, 100), dtype=np.float32)
    out = oracle.qshift(x, H, W, 1, 0.125)
    zero_ch = np.nonzero((out[0] == 0).any(axis=0))[0]
    assert zero_ch.min() == 0 and zero_ch.max() == 49
    g = out[0].reshape(H, W, 100)
    assert np.all(g[:, 0, :12] == 0) and np.all(g[:, 1:, :12] == 1)       # right shift group
    assert np.all(g[:, 2, 12:25] == 0) and np.all(g[:, :2, 12:25] == 1)   # left shift group
    assert np.all(g[0, :, 25:37] == 0) and np.all(g[1:, :, 25:37] == 1)   # down shift group
    assert np.all(g[2, :, 37:50] == 0) and np.all(g[:2, :, 37:50] == 1)   # up shift group
    assert np.all(g[..., 50:] == 1)


def test_qshift_identities():
    g = _rng(7)
    x = g.standard_normal((2, 20, 12)).astype(np.float32)
    np.testing.assert_array_equal(oracle.qshift(x, 4, 5, 0, 0.25), x)
    np.testing.assert_array_equal(oracle.qshift(x, 4, 5, 1, 0.0), x)
    x2 = g.standard_normal((1, 16, 8)).astype(np.float32)
    out = oracle.qshift(x2, 4, 4, 4, 0.25)
    assert np.all(out == 0)  # shift equal to the grid side zeroes all four groups (C = 4*C/4)


@pytest.mark.parametrize("shift,gamma", [(1, 0.26), (1, -0.01), (1, float("nan")), (-1, 0.25), (5, 0.25)])
def test_qshift_rejects_invalid(shift, gamma):
    x = np.zeros((1, 12, 8), dtype=np.float32)
    with pytest.raises(oracle.QShiftParamError):
        oracle.qshift(x, 3, 4, shift, gamma)


def test_fused_is_composition():
    g = _rng(8)
    H, W, C = 5, 6, 16
    k = g.standard_normal((2, H * W, C)).astype(np.float32).astype(np.float64)
    v = g.standard_normal((2, H * W, C)).astype(np.float32).astype(np.float64)
    w = g.uniform(-3, 3, C)
    u = g.standard_normal(C)
    y = oracle.biwkv_qshift(k, v, w, u, H, W, 1, 0.25, use_rnn=False)
    ks = _qshift_roll(k.astype(np.float32), H, W, 1, 0.25).astype(np.float64)
    vs = _qshift_roll(v.astype(np.float32), H, W, 1, 0.25).astype(np.float64)
    np.testing.assert_array_equal(y, oracle.biwkv_sum(ks, vs, w, u))
