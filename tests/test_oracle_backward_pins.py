"""Pins for the oracle's Bi-WKV gradients (Eq. (5) of the Vision-RWKV article, section "Linear
Complexity Bidirectional Attention"; the article states an O(TC) backward recurrence but does not
print it, so the gradients are derived from Eq. (5)).

The definition form and the linear-time form are pinned to central finite differences of the
forward oracle (itself pinned in test_oracle_pins.py), to exact identities of Eq. (5) (invariance
to a per-channel shift of k, affinity in v, homogeneity in v), to closed forms for T = 1 and 2,
and planted mistakes must fail them.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle


def _rand(seed, B, T, C, kstd=1.0, wr=5.0):
    g = np.random.Generator(np.random.PCG64(5000 + seed))
    k = g.standard_normal((B, T, C)) * kstd
    v = g.standard_normal((B, T, C))
    w = g.uniform(-wr, wr, C)
    u = g.standard_normal(C)
    gy = g.standard_normal((B, T, C))
    return k, v, w, u, gy


def _loss(k, v, w, u, gy):
    return float((oracle.biwkv_sum(k, v, w, u) * gy).sum())


def _fd_all(k, v, w, u, gy, h=1e-6):
    """Central finite differences of L = sum(g * y) for every input element (small sizes)."""
    out = []
    for arr_i in range(4):
        args = [k, v, w, u]
        base = args[arr_i]
        grad = np.empty_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            p = [a.copy() for a in args]
            m = [a.copy() for a in args]
            p[arr_i][idx] += h
            m[arr_i][idx] -= h
            grad[idx] = (_loss(*p, gy) - _loss(*m, gy)) / (2 * h)
        out.append(grad)
    return out  # dk, dv, dw, du


@pytest.mark.parametrize("B,T,C", [(1, 1, 2), (1, 2, 3), (2, 5, 2), (1, 9, 3), (2, 16, 2)])
def test_gradients_match_finite_differences(B, T, C):
    k, v, w, u, gy = _rand(T * 10 + C, B, T, C, kstd=1.5, wr=6.0)
    fk, fv, fw, fu = _fd_all(k, v, w, u, gy)
    for name, fn in (("sum", oracle.biwkv_backward_sum), ("rnn", oracle.biwkv_backward_rnn)):
        dk, dv, dw, du = fn(k, v, w, u, gy)
        np.testing.assert_allclose(dk, fk, rtol=1e-6, atol=1e-8, err_msg=name)
        np.testing.assert_allclose(dv, fv, rtol=1e-6, atol=1e-8, err_msg=name)
        np.testing.assert_allclose(dw, fw, rtol=1e-6, atol=1e-8, err_msg=name)
        np.testing.assert_allclose(du, fu, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("T,C,B", [(3, 2, 1), (17, 3, 2), (64, 4, 1), (200, 2, 1)])
def test_definition_equals_linear_time_form(T, C, B):
    k, v, w, u, gy = _rand(T, B, T, C, kstd=2.0, wr=8.0)
    a = oracle.biwkv_backward_sum(k, v, w, u, gy, with_scale=True)
    b = oracle.biwkv_backward_rnn(k, v, w, u, gy)
    for x, y, s in zip(a[:4], b, a[4:]):
        assert np.all(np.abs(x - y) <= 1e-10 * np.maximum(s, 1e-300) + 1e-300)


def test_exact_identities():
    """sum_i dk_i = 0 (y is unchanged by k + const), sum_i dv_i = sum_t g_t (y(v + b) = y + b) and
    sum_i v_i dv_i = sum_t g_t y_t (y(a v) = a y), per batch item and channel."""
    k, v, w, u, gy = _rand(3, 2, 40, 5, kstd=2.0, wr=8.0)
    dk, dv, _, _ = oracle.biwkv_backward_sum(k, v, w, u, gy)
    y = oracle.biwkv_sum(k, v, w, u)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=1), gy.sum(axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose((v * dv).sum(axis=1), (gy * y).sum(axis=1), rtol=1e-11, atol=1e-12)


def test_closed_forms_T1_T2():
    k, v, w, u, gy = _rand(4, 2, 1, 3)
    dk, dv, dw, du = oracle.biwkv_backward_sum(k, v, w, u, gy)
    np.testing.assert_array_equal(dv, gy)
    np.testing.assert_array_equal(dk, 0.0 * k)
    np.testing.assert_array_equal(dw, np.zeros(3))
    np.testing.assert_array_equal(du, np.zeros(3))
    k, v, w, u, gy = _rand(5, 2, 2, 3)
    _, _, dw, _ = oracle.biwkv_backward_sum(k, v, w, u, gy)
    np.testing.assert_array_equal(dw, np.zeros(3))  # T = 2: neighbours carry no decay


BACKWARD_MUTATIONS = {
    "dw_without_minus_one": ("const double dterm = term * (-((double)(dist - 1)) / Td);",
                             "const double dterm = term * (-((double)(dist)) / Td);"),
    "dk_uses_own_output": ("const double term = gp * (vc[i] - y[t]);", "const double term = gp * (vc[i] - y[i]);"),
    "du_from_all_terms": ("if (t == i) {\n                            duc += term;", "if (1) {\n                            duc += term;"),
    "rnn_prefix_suffix_swapped": ("dwc += bb[i] * qp[i] - d[i] * rp[i] + a[i] * qs[i] - cc[i] * rs[i];",
                                  "dwc += bb[i] * qs[i] - d[i] * rs[i] + a[i] * qp[i] - cc[i] * rp[i];"),
    "rnn_missing_bonus_in_dv": ("e[i] * (qp[i] + qs[i] + eu * q[i]);", "e[i] * (qp[i] + qs[i] + q[i]);"),
}


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTATIONS))
def test_backward_pins_catch_planted_mistakes(tmp_path, name):
    old, new = BACKWARD_MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "biwkv_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not found: {name}"
    c_path, so_path = tmp_path / f"{name}.c", tmp_path / f"{name}.so"
    c_path.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so_path))
    P, I = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_biwkv_backward_sum.argtypes = [P] * 5 + [I] * 3 + [P] * 8 + [ctypes.c_int]
    lib.oracle_biwkv_backward_rnn.argtypes = [P] * 5 + [I] * 3 + [P] * 4 + [ctypes.c_int]
    B, T, C = 1, 7, 2
    k, v, w, u, gy = _rand(77, B, T, C, kstd=1.5, wr=6.0)
    fd = _fd_all(k, v, w, u, gy)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    caught = False
    for fn in ("sum", "rnn"):
        dk, dv, dw, du = np.empty_like(k), np.empty_like(k), np.empty(C), np.empty(C)
        if fn == "sum":
            lib.oracle_biwkv_backward_sum(ptr(k), ptr(v), ptr(w), ptr(u), ptr(gy), B, T, C, ptr(dk), ptr(dv),
                                          ptr(dw), ptr(du), None, None, None, None, 1)
        else:
            lib.oracle_biwkv_backward_rnn(ptr(k), ptr(v), ptr(w), ptr(u), ptr(gy), B, T, C, ptr(dk), ptr(dv),
                                          ptr(dw), ptr(du), 1)
        for got, ref in zip((dk, dv, dw, du), fd):
            if not np.allclose(got, ref, rtol=1e-5, atol=1e-7):
                caught = True
    assert caught, f"planted mistake {name} went unnoticed"
