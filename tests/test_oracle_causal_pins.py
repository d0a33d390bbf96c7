"""Pins for the oracle's causal attention (the original RWKV form the Vision-RWKV article starts
from, section "Linear Complexity Bidirectional Attention": the sum stops at the token before the
current one; Bi-WKV raises that limit to T-1).

Reading: Eq. (5) with the decayed sum over i < t only, the same exponent -((t-1-i)/T) w + k_i and
the same self term e^{u+k_t}. Each test pins it to something other than its own formula: the
bidirectional oracle on a truncated sequence, scipy's softmax, closed forms, and invariants.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from tests.metrics import r3


def _rand(seed, B, T, C, kstd=1.0, wr=5.0, ustd=1.0):
    g = np.random.Generator(np.random.PCG64(2000 + seed))
    k = g.standard_normal((B, T, C)) * kstd
    v = g.standard_normal((B, T, C))
    w = g.uniform(-wr, wr, C)
    u = g.standard_normal(C) * ustd
    return k, v, w, u


@pytest.mark.parametrize("T,C,B", [(1, 3, 1), (2, 2, 2), (5, 3, 1), (17, 4, 2), (64, 3, 1)])
def test_causal_sum_equals_rnn(T, C, B):
    k, v, w, u = _rand(T, B, T, C, kstd=3.0, wr=8.0)
    y1, s1 = oracle.biwkv_causal_sum(k, v, w, u, with_scale=True)
    y2, s2 = oracle.biwkv_causal_rnn(k, v, w, u, with_scale=True)
    assert r3(y2, y1, s1) <= 1e-12
    np.testing.assert_allclose(s2, s1, rtol=1e-10)


@pytest.mark.parametrize("T", [2, 7, 30])
def test_causal_is_bidirectional_on_the_prefix(T):
    """Token t of the causal form is the last token of Bi-WKV over tokens 0..t (nothing follows it),
    with w rescaled so that Bi-WKV's division by t + 1 matches the causal division by T."""
    k, v, w, u = _rand(T + 1, 2, T, 4, kstd=2.0, wr=6.0)
    y = oracle.biwkv_causal_sum(k, v, w, u)
    for t in range(T):
        wp = w * (t + 1) / T
        yp = oracle.biwkv_sum(k[:, : t + 1], v[:, : t + 1], wp, u)
        np.testing.assert_allclose(y[:, t], yp[:, t], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T", [4, 33])
def test_causal_single_query_softmax(T):
    """Per channel and token, the causal form is softmax attention over tokens 0..t with a bias
    linear in the distance: scipy's softmax over a masked logit matrix."""
    k, v, w, u = _rand(T + 5, 1, T, 3, kstd=2.0, wr=6.0)
    d = np.subtract.outer(np.arange(T), np.arange(T)).astype(np.float64)  # t - i
    y_ref = np.empty((1, T, 3))
    for c in range(3):
        logits = -(d - 1.0) / T * w[c] + k[0, :, c][None, :]
        np.fill_diagonal(logits, u[c] + k[0, :, c])
        logits[d < 0] = -np.inf
        y_ref[0, :, c] = softmax(logits, axis=1) @ v[0, :, c]
    np.testing.assert_allclose(oracle.biwkv_causal_sum(k, v, w, u), y_ref, rtol=1e-12, atol=1e-13)


def test_causal_first_token_is_v():
    k, v, w, u = _rand(3, 2, 12, 5, kstd=3.0)
    for fn in (oracle.biwkv_causal_sum, oracle.biwkv_causal_rnn):
        np.testing.assert_allclose(fn(k, v, w, u)[:, 0], v[:, 0], rtol=2.3e-16, atol=0)


def test_causal_strong_decay_gives_two_tap():
    """w -> +inf: only the previous token (distance 1, no decay) and the self term survive."""
    T = 9
    k, v, _, u = _rand(4, 1, T, 3)
    y = oracle.biwkv_causal_sum(k, v, np.full(3, 1e5), u)
    ek, eu = np.exp(k), np.exp(u)
    num, den = eu * ek * v, eu * ek
    num[:, 1:] += ek[:, :-1] * v[:, :-1]
    den[:, 1:] += ek[:, :-1]
    np.testing.assert_allclose(y, num / den, rtol=1e-12)


def test_causal_ignores_the_future():
    k, v, w, u = _rand(6, 1, 20, 4, kstd=2.0)
    y = oracle.biwkv_causal_sum(k, v, w, u)
    k2, v2 = k.copy(), v.copy()
    k2[:, 11:] += 5.0
    v2[:, 11:] = -v2[:, 11:] * 3.0
    y2 = oracle.biwkv_causal_sum(k2, v2, w, u)
    np.testing.assert_array_equal(y2[:, :11], y[:, :11])
    assert not np.allclose(y2[:, 11:], y[:, 11:])


def test_causal_last_token_equals_bidirectional():
    k, v, w, u = _rand(7, 2, 25, 3, kstd=2.0, wr=7.0)
    np.testing.assert_allclose(oracle.biwkv_causal_sum(k, v, w, u)[:, -1],
                               oracle.biwkv_sum(k, v, w, u)[:, -1], rtol=1e-12, atol=1e-14)


CAUSAL_MUTATIONS = {
    "dropped_minus_one": ("-(((double)(t - 1 - i)) / Td) * wc", "-(((double)(t - i)) / Td) * wc"),
    "decay_sign_flipped": (": -(((double)(t - 1 - i)) / Td) * wc", ": (((double)(t - 1 - i)) / Td) * wc"),
    "future_included": ("for (int64_t i = 0; i <= t; ++i)", "for (int64_t i = 0; i <= t + (t + 1 < T); ++i)"),
    "bonus_dropped": ("(i == t) ? uc + kc[i]", "(i == t) ? kc[i]"),
    "rnn_self_term_in_state": ("out[(b * T + t) * C + c] = (A + E * vc[t]) / (Cs + E);",
                               "out[(b * T + t) * C + c] = (A + exp(kc[t] - kappa) * vc[t] + E * vc[t]) / (Cs + exp(kc[t] - kappa) + E);"),
}


@pytest.mark.parametrize("name", sorted(CAUSAL_MUTATIONS))
def test_causal_pins_catch_planted_mistakes(tmp_path, name):
    """A plausible mistake planted in a temporary copy of the oracle source (CPU only) breaks the
    prefix relation to the unmodified bidirectional oracle."""
    import ctypes
    import os
    import subprocess

    old, new = CAUSAL_MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "biwkv_oracle.c")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {name}"
    c_path, so_path = tmp_path / f"{name}.c", tmp_path / f"{name}.so"
    c_path.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so_path))
    P, I = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_biwkv_causal_sum.argtypes = [P, P, P, P, I, I, I, P, P, ctypes.c_int]
    lib.oracle_biwkv_causal_rnn.argtypes = [P, P, P, P, I, I, I, P, P, ctypes.c_int]
    T, C = 9, 3
    k, v, w, u = _rand(40, 1, T, C, kstd=1.5, wr=6.0)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    caught = False
    for fn in ("sum", "rnn"):
        out = np.empty((1, T, C))
        if fn == "sum":
            lib.oracle_biwkv_causal_sum(ptr(k), ptr(v), ptr(w), ptr(u), 1, T, C, ptr(out), None, 1)
        else:
            lib.oracle_biwkv_causal_rnn(ptr(k), ptr(v), ptr(w), ptr(u), 1, T, C, ptr(out), None, 1)
        for t in range(T):
            ref = oracle.biwkv_sum(k[:, : t + 1], v[:, : t + 1], w * (t + 1) / T, u)[:, t]
            if not np.allclose(out[:, t], ref, rtol=1e-9, atol=1e-12):
                caught = True
    assert caught, f"planted mistake {name} went unnoticed"
