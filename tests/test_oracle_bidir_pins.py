"""Pins for the oracle's bidirectional shift: the Q-Shift that the Vision-RWKV article's MAE
paragraph (section "MAE pre-training") makes bidirectional so that the model takes sparse inputs.

Reading: on the sequence of visible tokens (no H x W grid), the channel groups that the q_shift
function of "LinXin's Blog" Vision-RWKV notes moves right or down take the earlier token n - s,
the groups it moves left or up take the later token n + s; zero fill at the ends, remainder
copied, values moved as raw bits.

Each test pins the oracle to something other than its own loop: a hand-derived fixture, the
already pinned grid Q-Shift on a 1 x N row and an N x 1 column, a slice formulation written
independently, zero counts, identities; planted mistakes must fail them.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bounds(C, gamma):
    return [int(C * gamma * j) for j in (1, 2, 3, 4)]


def _bidir_slices(bits, shift, gamma):
    """Independent formulation: whole-axis slices per channel group."""
    B, N, C = bits.shape
    g = _bounds(C, gamma)
    s = shift
    out = np.zeros_like(bits)
    out[:, :, g[3]:] = bits[:, :, g[3]:]
    for lo, hi, earlier in ((0, g[0], True), (g[0], g[1], False), (g[1], g[2], True), (g[2], g[3], False)):
        if hi <= lo or s >= N and s > 0:
            continue
        if s == 0:
            out[:, :, lo:hi] = bits[:, :, lo:hi]
        elif earlier:
            out[:, s:, lo:hi] = bits[:, : N - s, lo:hi]
        else:
            out[:, : N - s, lo:hi] = bits[:, s:, lo:hi]
    return out


def _random_bits(seed, B, N, C):
    g = np.random.Generator(np.random.PCG64(7000 + seed))
    bits = g.integers(0, 2**32, size=(B, N, C), dtype=np.uint64).astype(np.uint32)
    if N and C:
        bits[0, 0, : min(C, 4)] = [0x7FC00000, 0x7F800001, 0x00000001, 0x80000000][: min(C, 4)]
    return bits


def test_bidir_hand_fixture():
    meta, rows = {}, []
    with open(os.path.join(GOLDEN, "qshift_bidir_hand_N5_C5.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0].isalpha():
                meta[parts[0]] = float(parts[1])
            else:
                rows.append([float(p) for p in parts])
    N, C = int(meta["N"]), int(meta["C"])
    x = np.array([[1000 + 100 * c + n for c in range(C)] for n in range(N)], dtype=np.float32)[None]
    out = oracle.qshift_bidir(x, int(meta["shift"]), meta["gamma"])
    exp = np.array([r[1:] for r in rows], dtype=np.float32)[None]
    np.testing.assert_array_equal(out, exp)


@pytest.mark.parametrize("N,C,gamma", [(49, 384, 0.25), (7, 10, 0.2), (30, 100, 0.125), (1, 8, 0.25), (5, 17, 0.25)])
def test_bidir_is_grid_qshift_on_a_row_and_a_column(N, C, gamma):
    """With shift 1 the horizontal groups move exactly as Q-Shift on a 1 x N grid and the vertical
    groups as Q-Shift on an N x 1 grid (the two ways a grid can be a single sequence)."""
    bits = _random_bits(N + C, 2, N, C)
    x = bits.view(np.float32)
    g = _bounds(C, gamma)
    out = oracle.qshift_bidir(x, 1, gamma).view(np.uint32)
    row = oracle.qshift(x, 1, N, 1, gamma).view(np.uint32)
    col = oracle.qshift(x, N, 1, 1, gamma).view(np.uint32)
    np.testing.assert_array_equal(out[..., : g[1]], row[..., : g[1]])
    np.testing.assert_array_equal(out[..., g[1]: g[3]], col[..., g[1]: g[3]])
    np.testing.assert_array_equal(out[..., g[3]:], bits[..., g[3]:])


@pytest.mark.parametrize("N,C,shift,gamma", [
    (49, 384, 1, 0.25), (1024, 64, 1, 0.25), (7, 10, 2, 0.2), (30, 100, 3, 0.125), (5, 9, 5, 0.25),
    (6, 13, 0, 0.25), (12, 16, 4, 0.0), (3, 4, 2, 0.25)])
def test_bidir_bitwise_against_slice_formulation(N, C, shift, gamma):
    bits = _random_bits(N * 3 + C + shift, 2, N, C)
    out = oracle.qshift_bidir(bits.view(np.float32), shift, gamma).view(np.uint32)
    np.testing.assert_array_equal(out, _bidir_slices(bits, shift, gamma))


@pytest.mark.parametrize("N,C,shift,gamma", [(49, 384, 1, 0.25), (30, 100, 3, 0.125), (9, 13, 9, 0.2)])
def test_bidir_zero_count(N, C, shift, gamma):
    """Each shifted channel loses exactly min(s, N) tokens at one end: s * g4 zeros per item."""
    x = np.ones((2, N, C), dtype=np.float32)
    out = oracle.qshift_bidir(x, shift, gamma)
    g4 = _bounds(C, gamma)[3]
    assert (out == 0).sum() == 2 * shift * g4
    assert (out != 0).all(axis=1)[:, g4:].all()


def test_bidir_identities():
    bits = _random_bits(1, 2, 11, 12)
    x = bits.view(np.float32)
    np.testing.assert_array_equal(oracle.qshift_bidir(x, 0, 0.25).view(np.uint32), bits)
    np.testing.assert_array_equal(oracle.qshift_bidir(x, 3, 0.0).view(np.uint32), bits)
    out = oracle.qshift_bidir(x, 11, 0.25).view(np.uint32)
    assert (out[..., :12] == 0).all()
    # reversing the tokens exchanges the earlier- and later-taking groups (equal sizes at C = 12)
    g = _bounds(12, 0.25)
    rev = oracle.qshift_bidir(bits[:, ::-1].copy().view(np.float32), 2, 0.25).view(np.uint32)[:, ::-1]
    fwd = oracle.qshift_bidir(x, 2, 0.25).view(np.uint32)
    swap = np.r_[g[0]:g[1], 0:g[0], g[2]:g[3], g[1]:g[2], g[3]:12]
    rev_sw = oracle.qshift_bidir(bits[:, ::-1][..., swap].copy().view(np.float32), 2, 0.25).view(np.uint32)
    np.testing.assert_array_equal(rev_sw[:, ::-1][..., np.argsort(swap)], fwd)
    assert not np.array_equal(rev, fwd)


@pytest.mark.parametrize("shift,gamma", [(-1, 0.25), (12, 0.25), (1, 0.26), (1, -0.1), (1, float("nan"))])
def test_bidir_rejects_invalid(shift, gamma):
    x = np.zeros((1, 11, 8), dtype=np.float32)
    with pytest.raises(oracle.QShiftParamError):
        oracle.qshift_bidir(x, shift, gamma)


BIDIR_MUTATIONS = {
    "first_token_kept": ("valid = n >= s;\n                    } else {", "valid = n > s;\n                    } else {"),
    "halves_instead_of_quarters": ("const int earlier = c < g1 || (c >= g2 && c < g3);", "const int earlier = c < g2;"),
    "later_groups_look_back": ("src = n + s;\n                        valid = n < N - s;",
                               "src = n - s;\n                        valid = n >= s;"),
    "remainder_shifted": ("if (c < g4) {\n                    const int earlier", "if (c < C) {\n                    const int earlier"),
}


@pytest.mark.parametrize("name", sorted(BIDIR_MUTATIONS))
def test_bidir_pins_catch_planted_mistakes(tmp_path, name):
    old, new = BIDIR_MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "biwkv_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not found: {name}"
    c_path, so_path = tmp_path / f"{name}.c", tmp_path / f"{name}.so"
    c_path.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so_path))
    P, I = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_qshift_bidir.argtypes = [P, P, I, I, I, I, ctypes.c_double]
    caught = False
    for N, C, shift, gamma in ((7, 10, 2, 0.2), (30, 100, 3, 0.125), (49, 384, 1, 0.25)):
        bits = _random_bits(N + C, 2, N, C)
        out = np.empty_like(bits)
        lib.oracle_qshift_bidir(bits.ctypes.data_as(P), out.ctypes.data_as(P), 2, N, C, shift, gamma)
        if not np.array_equal(out, _bidir_slices(bits, shift, gamma)):
            caught = True
    assert caught, f"planted mistake {name} went unnoticed"
