"""Pins for the oracle's Eq. (2) gate and Eq. (9) mixing ("OpenGVLab&港中文&复旦&南大&清华提出
Vision-RWKV Backbone": spatial-mix block, Eq. (2); Quad-Directional Token Shift, Eq. (9)).

Reading of Eq. (9): the equation as printed, X + (1 - mu) X-dagger per mixing vector (the prose
calls it an interpolation; see the design notes). Each test pins the oracle to something other
than its own formula: scipy's logistic function, closed forms and limits, and a per-element loop.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def _g(seed):
    return np.random.Generator(np.random.PCG64(3000 + seed))


def test_sigmoid_matches_scipy():
    x = np.concatenate([np.linspace(-50, 50, 2001), [-745.0, 0.0, 745.0, 1e-300]])
    np.testing.assert_allclose(oracle.sigmoid(x), expit(x), rtol=1e-15, atol=1e-300)


def test_gate_limits():
    g = _g(1)
    B, T, C = 2, 13, 5
    k, v = g.standard_normal((B, T, C)), g.standard_normal((B, T, C))
    w, u = g.uniform(-5, 5, C), g.standard_normal(C)
    y = oracle.biwkv_rnn(k, v, w, u)
    np.testing.assert_array_equal(oracle.biwkv_gated(k, v, np.full((B, T, C), 40.0), w, u), y)
    np.testing.assert_array_equal(oracle.biwkv_gated(k, v, np.zeros((B, T, C)), w, u), 0.5 * y)
    r = g.standard_normal((B, T, C)) * 3
    np.testing.assert_allclose(oracle.biwkv_gated(k, v, r, w, u), expit(r) * oracle.biwkv_sum(k, v, w, u),
                               rtol=1e-12, atol=1e-15)


def test_mix_limits_and_loop():
    g = _g(2)
    B, H, W, C, s, gam = 2, 3, 4, 10, 1, 0.2
    x = g.standard_normal((B, H * W, C)).astype(np.float32)
    mu = np.stack([np.ones(C), np.zeros(C), g.uniform(0, 1, C)])
    out = oracle.qshift_mix(x, mu, H, W, s, gam)
    np.testing.assert_array_equal(out[0], x.astype(np.float64))
    xd = oracle.qshift_f64(x, H, W, s, gam)
    np.testing.assert_array_equal(out[1], x + xd)
    # per-element loop over the grid, written from the q_shift description (groups at int(C*g*j))
    bounds = [int(C * gam * j) for j in (1, 2, 3, 4)]
    ref = np.empty((B, H * W, C))
    for b in range(B):
        for h in range(H):
            for ww in range(W):
                for c in range(C):
                    if c < bounds[0]:
                        hs, ws = h, ww - s
                    elif c < bounds[1]:
                        hs, ws = h, ww + s
                    elif c < bounds[2]:
                        hs, ws = h - s, ww
                    elif c < bounds[3]:
                        hs, ws = h + s, ww
                    else:
                        hs, ws = h, ww
                    src = float(x[b, hs * W + ws, c]) if (0 <= hs < H and 0 <= ws < W) else 0.0
                    ref[b, h * W + ww, c] = float(x[b, h * W + ww, c]) + (1.0 - mu[2, c]) * src
    np.testing.assert_allclose(out[2], ref, rtol=1e-15, atol=0)


def test_mix_rejects_bad_mu():
    x = np.zeros((1, 4, 8), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.qshift_mix(x, np.zeros(8), 2, 2)
