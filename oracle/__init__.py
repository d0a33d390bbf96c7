"""Plain CPU float64 oracle for Bi-WKV and Q-Shift (ctypes wrapper around biwkv_oracle.c).

TEST INFRASTRUCTURE ONLY: the product path never imports this package. Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it. It shares no
code with the HIP library.

Functions follow the pages (cited by title and equation):

* ``biwkv_sum``      — Eq. (5) summation form, "OpenGVLab&港中文&复旦&南大&清华提出Vision-RWKV
  Backbone", section "Linear Complexity Bidirectional Attention".
* ``biwkv_rnn``      — Eq. (6)-(7) RNN form with four hidden states, two sweeps (same section).
* ``biwkv_rnn_literal`` — the same section's prose update (add/remove one term, multiply/divide by
  e^{-w/T}) read literally; small T only.
* ``qshift``         — the q_shift function of "LinXin's Blog" Vision-RWKV notes (token shift on
  the H x W grid, groups at int(C*gamma*j), zero fill, remainder copied).
* ``biwkv_qshift``   — the fused composition Bi-WKV(X†(k), X†(v)).
* ``biwkv_backward_sum`` / ``biwkv_backward_rnn`` — gradients of Eq. (5) (the article says the
  backward pass is an O(TC) recurrence; its formulas are not on the pages): the definition written
  out, and the linear-time form as decayed prefix / suffix sums.
* ``sigmoid`` / ``biwkv_gated`` — Eq. (2) of the same article: the attention output gated by
  sigma(R) (elementwise) before the output projection.
* ``qshift_mix``     — Eq. (9) as printed: X + (1 - mu) X-dagger for each mixing vector mu.
* ``qshift_bidir``   — the bidirectional shift of the same article's MAE paragraph (Q-Shift on a
  sparse token sequence): the groups that Q-Shift moves right or down take token n - s, the
  groups it moves left or up take token n + s; zero fill, remainder copied.
* ``biwkv_causal_sum`` / ``biwkv_causal_rnn`` — the causal attention Bi-WKV is derived from (the
  original RWKV attention, which the same section says stops at the current token): Eq. (5)
  with the decayed sum over i < t only, and Eq. (6)-(7) with b = d = 0.

All arrays are numpy, [B, T, C] C-contiguous. Floating inputs are widened to float64 (exact for
fp32 and bf16 values).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "biwkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain IEEE float64: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_biwkv_sum.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P, ctypes.c_int]
        lib.oracle_biwkv_rnn.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, ctypes.c_int]
        lib.oracle_biwkv_rnn_literal.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P]
        lib.oracle_qshift.argtypes = [_P, _P, _I64, _I64, _I64, _I64, _I64, ctypes.c_double]
        lib.oracle_qshift_bidir.argtypes = [_P, _P, _I64, _I64, _I64, _I64, ctypes.c_double]
        lib.oracle_biwkv_causal_sum.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, ctypes.c_int]
        lib.oracle_biwkv_causal_rnn.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, ctypes.c_int]
        lib.oracle_biwkv_backward_sum.argtypes = [_P] * 5 + [_I64] * 3 + [_P] * 8 + [ctypes.c_int]
        lib.oracle_biwkv_backward_rnn.argtypes = [_P] * 5 + [_I64] * 3 + [_P] * 4 + [ctypes.c_int]
        for f in (lib.oracle_biwkv_sum, lib.oracle_biwkv_rnn, lib.oracle_biwkv_rnn_literal, lib.oracle_qshift, lib.oracle_qshift_bidir,
                  lib.oracle_biwkv_causal_sum, lib.oracle_biwkv_causal_rnn, lib.oracle_biwkv_backward_sum,
                  lib.oracle_biwkv_backward_rnn):
            f.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_bitc(k, v, w, u):
    k, v, w, u = _f64(k), _f64(v), _f64(w).reshape(-1), _f64(u).reshape(-1)
    if k.ndim != 3 or v.shape != k.shape:
        raise ValueError("k and v must both be [B, T, C]")
    B, T, C = k.shape
    if w.shape != (C,) or u.shape != (C,):
        raise ValueError("w and u must be [C]")
    return k, v, w, u, B, T, C


def biwkv_sum(k, v, w, u, rows=None, with_scale=False, threads=0):
    """Eq. (5) summation form. ``rows``: optional token indices (output is then [B, len(rows), C])."""
    k, v, w, u, B, T, C = _check_bitc(k, v, w, u)
    if rows is None:
        rows_arr, nrows, rows_p = None, T, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        nrows, rows_p = rows_arr.size, _ptr(rows_arr)
    out = np.empty((B, nrows, C), dtype=np.float64)
    scale = np.empty_like(out) if with_scale else None
    rc = _load().oracle_biwkv_sum(_ptr(k), _ptr(v), _ptr(w), _ptr(u), B, T, C, rows_p, nrows,
                                  _ptr(out), _ptr(scale) if scale is not None else None, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_biwkv_sum failed ({rc})")
    return (out, scale) if with_scale else out


def biwkv_rnn(k, v, w, u, with_scale=False, threads=0):
    """Eq. (6)-(7) RNN form, two sweeps over the four hidden states."""
    k, v, w, u, B, T, C = _check_bitc(k, v, w, u)
    out = np.empty((B, T, C), dtype=np.float64)
    scale = np.empty_like(out) if with_scale else None
    rc = _load().oracle_biwkv_rnn(_ptr(k), _ptr(v), _ptr(w), _ptr(u), B, T, C, _ptr(out),
                                  _ptr(scale) if scale is not None else None, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_biwkv_rnn failed ({rc})")
    return (out, scale) if with_scale else out


def biwkv_rnn_literal(k, v, w, u):
    """The literal single-sweep prose recurrence (small T only)."""
    k, v, w, u, B, T, C = _check_bitc(k, v, w, u)
    out = np.empty((B, T, C), dtype=np.float64)
    rc = _load().oracle_biwkv_rnn_literal(_ptr(k), _ptr(v), _ptr(w), _ptr(u), B, T, C, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_biwkv_rnn_literal failed ({rc})")
    return out


def biwkv_causal_sum(k, v, w, u, with_scale=False, threads=0):
    """Causal attention (sum stops before the current token; same exponent convention as Eq. (5))."""
    k, v, w, u, B, T, C = _check_bitc(k, v, w, u)
    out = np.empty((B, T, C), dtype=np.float64)
    scale = np.empty_like(out) if with_scale else None
    rc = _load().oracle_biwkv_causal_sum(_ptr(k), _ptr(v), _ptr(w), _ptr(u), B, T, C, _ptr(out),
                                         _ptr(scale) if scale is not None else None, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_biwkv_causal_sum failed ({rc})")
    return (out, scale) if with_scale else out


def biwkv_causal_rnn(k, v, w, u, with_scale=False, threads=0):
    """Causal attention in RNN form: prefix states a, c of Eq. (6) and Eq. (7) with b = d = 0."""
    k, v, w, u, B, T, C = _check_bitc(k, v, w, u)
    out = np.empty((B, T, C), dtype=np.float64)
    scale = np.empty_like(out) if with_scale else None
    rc = _load().oracle_biwkv_causal_rnn(_ptr(k), _ptr(v), _ptr(w), _ptr(u), B, T, C, _ptr(out),
                                         _ptr(scale) if scale is not None else None, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_biwkv_causal_rnn failed ({rc})")
    return (out, scale) if with_scale else out


class QShiftParamError(ValueError):
    """Raised for the parameter combinations the q_shift listing rejects."""


def qshift(x, H, W, shift=1, gamma=0.25):
    """Q-Shift X† on a [B, H*W, C] array of 4-byte elements; returns the same dtype, bit for bit."""
    x = np.ascontiguousarray(x)
    if x.ndim != 3 or x.dtype.itemsize != 4:
        raise ValueError("x must be a [B, N, C] array of 4-byte elements")
    B, N, C = x.shape
    if N != H * W:
        raise ValueError("N must equal H * W")
    bits = x.view(np.uint32)
    out = np.empty_like(bits)
    rc = _load().oracle_qshift(_ptr(bits), _ptr(out), B, H, W, C, int(shift), float(gamma))
    if rc == -2:
        raise QShiftParamError(f"invalid shift={shift} / gamma={gamma} for a {H}x{W} grid")
    if rc != 0:
        raise RuntimeError(f"oracle_qshift failed ({rc})")
    return out.view(x.dtype)


def qshift_f64(x, H, W, shift=1, gamma=0.25):
    """Q-Shift of a float64 array, done on its float32 bit patterns (values must be fp32-exact)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64), equal_nan=True):
        raise ValueError("qshift_f64 needs values exactly representable in float32")
    return qshift(x32, H, W, shift, gamma).astype(np.float64)


def qshift_bidir(x, shift=1, gamma=0.25):
    """Bidirectional shift of a [B, N, C] array of 4-byte elements along the token axis (the
    MAE form of Q-Shift); returns the same dtype, bit for bit."""
    x = np.ascontiguousarray(x)
    if x.ndim != 3 or x.dtype.itemsize != 4:
        raise ValueError("x must be a [B, N, C] array of 4-byte elements")
    B, N, C = x.shape
    bits = x.view(np.uint32)
    out = np.empty_like(bits)
    rc = _load().oracle_qshift_bidir(_ptr(bits), _ptr(out), B, N, C, int(shift), float(gamma))
    if rc == -2:
        raise QShiftParamError(f"invalid shift={shift} / gamma={gamma} for {N} tokens")
    if rc != 0:
        raise RuntimeError(f"oracle_qshift_bidir failed ({rc})")
    return out.view(x.dtype)


def qshift_bidir_f64(x, shift=1, gamma=0.25):
    """The bidirectional shift of a float64 array, on its float32 bit patterns (fp32-exact values)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64), equal_nan=True):
        raise ValueError("qshift_bidir_f64 needs values exactly representable in float32")
    return qshift_bidir(x32, shift, gamma).astype(np.float64)


def biwkv_backward_sum(k, v, w, u, g, with_scale=False, threads=0):
    """Gradients of Eq. (5) from the definition (quadratic): returns dk, dv [B, T, C] and dw, du [C]
    (summed over the batch); with_scale also returns the sums of absolute terms of each."""
    k, v, w, u, B, T, C = _check_bitc(k, v, w, u)
    g = _f64(g)
    if g.shape != k.shape:
        raise ValueError("g must be [B, T, C]")
    dk, dv = np.empty_like(k), np.empty_like(k)
    dw, du = np.empty(C), np.empty(C)
    sc = [np.empty_like(k), np.empty_like(k), np.empty(C), np.empty(C)] if with_scale else [None] * 4
    rc = _load().oracle_biwkv_backward_sum(_ptr(k), _ptr(v), _ptr(w), _ptr(u), _ptr(g), B, T, C,
                                           _ptr(dk), _ptr(dv), _ptr(dw), _ptr(du),
                                           *[(_ptr(a) if a is not None else None) for a in sc], int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_biwkv_backward_sum failed ({rc})")
    return (dk, dv, dw, du, *sc) if with_scale else (dk, dv, dw, du)


def biwkv_backward_rnn(k, v, w, u, g, threads=0):
    """The same gradients in linear time (decayed prefix / suffix sums): dk, dv, dw, du."""
    k, v, w, u, B, T, C = _check_bitc(k, v, w, u)
    g = _f64(g)
    if g.shape != k.shape:
        raise ValueError("g must be [B, T, C]")
    dk, dv = np.empty_like(k), np.empty_like(k)
    dw, du = np.empty(C), np.empty(C)
    rc = _load().oracle_biwkv_backward_rnn(_ptr(k), _ptr(v), _ptr(w), _ptr(u), _ptr(g), B, T, C,
                                           _ptr(dk), _ptr(dv), _ptr(dw), _ptr(du), int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_biwkv_backward_rnn failed ({rc})")
    return dk, dv, dw, du


def sigmoid(x):
    """The logistic function of Eq. (2)'s gate (sigma), in float64: 1 / (1 + e^{-x})."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def biwkv_gated(k, v, r, w, u, with_scale=False, threads=0, use_sum=False):
    """Eq. (2)'s gated attention output before the output projection: sigma(R) * Bi-WKV(K, V)
    ("OpenGVLab&港中文&复旦&南大&清华提出Vision-RWKV Backbone", spatial-mix block, Eq. (2)).
    Bi-WKV from the RNN form, or from the summation form (use_sum: any w, small sizes)."""
    fn = biwkv_sum if use_sum else biwkv_rnn
    y, s = fn(k, v, w, u, with_scale=True, threads=threads)
    gate = sigmoid(r)
    return (gate * y, gate * s) if with_scale else gate * y


def qshift_mix(x, mu, H, W, shift=1, gamma=0.25):
    """Eq. (9) as printed, once per mixing vector: out[j] = X + (1 - mu[j]) * X-dagger, with
    X-dagger the q_shift gather (values must be fp32-exact); float64 result [J, B, N, C]."""
    x = np.asarray(x, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    if mu.ndim != 2 or mu.shape[1] != x.shape[2]:
        raise ValueError("mu must be [J, C]")
    xd = qshift_f64(x, H, W, shift, gamma)
    return np.stack([x + (1.0 - mu[j])[None, None, :] * xd for j in range(mu.shape[0])])


def biwkv_qshift(k, v, w, u, H, W, shift=1, gamma=0.25, use_rnn=True, with_scale=False, threads=0):
    """Fused path: Bi-WKV(X†(k), X†(v)) with T = H*W; zero-filled sources enter as 0."""
    ks = qshift_f64(k, H, W, shift, gamma)
    vs = qshift_f64(v, H, W, shift, gamma)
    fn = biwkv_rnn if use_rnn else biwkv_sum
    return fn(ks, vs, w, u, with_scale=with_scale, threads=threads)
