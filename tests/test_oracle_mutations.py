"""The oracle's pins have teeth: plausible mistakes planted in a temporary copy of the oracle's C
source (on the CPU only) must each be caught by a hand-derived fixture or the independent
Q-Shift formulation. The committed oracle itself is never modified.
"""
import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import _qshift_roll, _read_biwkv_cases

SRC = os.path.join(os.path.dirname(oracle.__file__), "biwkv_oracle.c")

BIWKV_MUTATIONS = {
    "dropped_minus_one": ("((double)(dist - 1)) / Td", "((double)(dist)) / Td"),
    "decay_sign_flipped": ("si = -(((double)(dist - 1)) / Td) * wc", "si = (((double)(dist - 1)) / Td) * wc"),
    "no_division_by_T": ("((double)(dist - 1)) / Td) * wc", "((double)(dist - 1))) * wc"),
    "bonus_dropped": ("si = uc + kc[i];", "si = kc[i];"),
    "key_dropped_from_neighbours": ("* wc + kc[i];", "* wc;"),
    "rnn_no_decay_forward": ("A = lam * A + e * vc[t];", "A = A + e * vc[t];"),
    "rnn_decay_inverted": ("const double lam = exp(-w[c] / (double)T);", "const double lam = exp(w[c] / (double)T);"),
    "rnn_self_term_in_state": ("aa[t] = A;", "aa[t] = A + exp(kc[t] - kappa) * vc[t];"),
}

QSHIFT_MUTATIONS = {
    "right_border_off_by_one": ("valid = wc >= s;", "valid = wc > s;"),
    "left_shift_wrong_way": ("sw = wc + s;", "sw = wc - s;"),
    "down_up_swapped": ("sh = h - s;", "sh = h + s;"),
    "group_bound_rounding": ("return (int64_t)x;", "return (int64_t)(x + 0.5);"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new)
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"{name}.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so_path))
    P, I = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_biwkv_sum.argtypes = [P, P, P, P, I, I, I, P, I, P, P, ctypes.c_int]
    lib.oracle_biwkv_rnn.argtypes = [P, P, P, P, I, I, I, P, P, ctypes.c_int]
    lib.oracle_qshift.argtypes = [P, P, I, I, I, I, I, ctypes.c_double]
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _fixture_fails(lib):
    for case in _read_biwkv_cases():
        T = int(case["T"])
        k = np.ascontiguousarray(np.array(case["k"], dtype=np.float64))
        v = np.ascontiguousarray(np.array(case["v"], dtype=np.float64))
        w = np.array([case["w"]])
        u = np.array([case["u"]])
        want = np.array([float(Fraction(y)) if isinstance(y, str) else y for y in case["y"]])
        for fn in ("sum", "rnn"):
            out = np.empty(T)
            if fn == "sum":
                lib.oracle_biwkv_sum(_ptr(k), _ptr(v), _ptr(w), _ptr(u), 1, T, 1, None, T, _ptr(out), None, 1)
            else:
                lib.oracle_biwkv_rnn(_ptr(k), _ptr(v), _ptr(w), _ptr(u), 1, T, 1, _ptr(out), None, 1)
            if not np.allclose(out, want, rtol=1e-12, atol=0):
                return True
    return False


@pytest.mark.parametrize("name", sorted(BIWKV_MUTATIONS))
def test_biwkv_mutation_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name, *BIWKV_MUTATIONS[name])
    assert _fixture_fails(lib), f"mutation {name} slipped past the hand-derived fixtures"


@pytest.mark.parametrize("name", sorted(QSHIFT_MUTATIONS))
def test_qshift_mutation_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name, *QSHIFT_MUTATIONS[name])
    caught = False
    for (H, W, C, s, g) in [(14, 14, 384, 1, 0.25), (5, 7, 100, 2, 0.125), (4, 4, 17, 3, 0.25)]:
        bits = np.random.Generator(np.random.PCG64(H * W + C)).integers(
            1, 2**31, size=(1, H * W, C), dtype=np.uint64).astype(np.uint32)
        out = np.empty_like(bits)
        lib.oracle_qshift(_ptr(bits), _ptr(out), 1, H, W, C, s, g)
        if not np.array_equal(out, _qshift_roll(bits, H, W, s, g)):
            caught = True
    assert caught, f"mutation {name} slipped past the independent Q-Shift formulation"


def test_unmutated_copy_passes(tmp_path):
    lib = _build_mutant(tmp_path, "identity", "#include <math.h>", "#include <math.h>")
    assert not _fixture_fails(lib)
