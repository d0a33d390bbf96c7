"""The C ABI of libbiwkv on the host: it loads, exports what include/biwkv.h declares, and rejects
bad arguments before any device work. No kernel runs here (no GPU is needed); pointers below are
never dereferenced because validation only looks at their values."""
import ctypes
import math

import pytest

import linear_complexity_vision_amd as lib


@pytest.fixture(scope="module")
def L():
    if not __import__("os").path.exists(lib.LIB_PATH):
        pytest.skip("libbiwkv.so is not built (run __graft_entry__.build())")
    return lib.load_library()


def test_every_declared_symbol_is_exported(L):
    names = lib.header_symbols()
    assert {"biwkv_forward", "qshift", "biwkv_qshift_forward", "biwkv_status_string",
            "biwkv_last_hip_error", "biwkv_stream_fault_flags", "biwkv_version"} <= set(names)
    for name in names:
        assert hasattr(L, name), f"{name} is declared in include/biwkv.h but not exported"


def test_status_codes_have_messages(L):
    codes = lib.status_codes()
    assert codes["BIWKV_OK"] == 0
    for name, code in codes.items():
        if name.startswith("BIWKV_ERR_"):
            assert code < 0
            assert lib.status_string(code) != "unknown status", name
    assert lib.status_string(12345) == "unknown status"
    assert L.biwkv_version() >= 100


# fake device addresses: distinct, 16-byte aligned, never dereferenced on the host
K, V, WP, UP, OUT = 0x10000000, 0x20000000, 0x30000000, 0x30001000, 0x40000000


def _fwd(L, k=K, v=V, w=WP, u=UP, out=OUT, B=2, T=8, C=4, dtype=lib.F32):
    return L.biwkv_forward(k, v, w, u, out, B, T, C, dtype, None)


def _fused(L, k=K, v=V, w=WP, u=UP, out=OUT, B=1, H=2, W=4, C=4, shift=1, gamma=0.25, dtype=lib.BF16):
    return L.biwkv_qshift_forward(k, v, w, u, out, B, H, W, C, shift, gamma, dtype, None)


def _qs(L, x=K, out=OUT, B=1, H=2, W=4, C=4, shift=1, gamma=0.25):
    return L.qshift(x, out, B, H, W, C, shift, gamma, None)


def _code(name):
    return lib.status_codes()[name]


def test_biwkv_forward_validation(L):
    assert _fwd(L, dtype=7) == _code("BIWKV_ERR_DTYPE")
    assert _fwd(L, k=None) == _code("BIWKV_ERR_NULL")
    assert _fwd(L, out=None) == _code("BIWKV_ERR_NULL")
    assert _fwd(L, w=None) == _code("BIWKV_ERR_NULL")
    assert _fwd(L, B=-1) == _code("BIWKV_ERR_SHAPE")
    assert _fwd(L, T=-3) == _code("BIWKV_ERR_SHAPE")
    assert _fwd(L, B=1 << 40, T=1 << 40, C=1 << 40) == _code("BIWKV_ERR_SHAPE")  # overflow
    assert _fwd(L, k=K + 1, dtype=lib.BF16) == _code("BIWKV_ERR_ALIGN")
    assert _fwd(L, k=K + 2, dtype=lib.F32) == _code("BIWKV_ERR_ALIGN")
    assert _fwd(L, out=K) == _code("BIWKV_ERR_ALIAS")
    assert _fwd(L, out=V + 8) == _code("BIWKV_ERR_ALIAS")
    assert _fwd(L, out=WP - 8) == _code("BIWKV_ERR_ALIAS")


def test_empty_calls_succeed_without_a_device(L):
    assert _fwd(L, B=0) == 0
    assert _fwd(L, T=0, k=None, v=None, out=None) == 0
    assert _fused(L, H=0, shift=0) == 0  # (a shift larger than an empty grid is rejected)
    assert _qs(L, C=0, x=None, out=None) == 0


def test_qshift_parameter_validation(L):
    bad = _code("BIWKV_ERR_PARAM")
    for shift, gamma in [(1, 0.3), (1, -0.1), (1, math.nan), (-1, 0.25), (3, 0.25), (5, 0.0)]:
        assert _qs(L, shift=shift, gamma=gamma) == bad, (shift, gamma)
        assert _fused(L, shift=shift, gamma=gamma) == bad, (shift, gamma)
    assert _qs(L, H=-1) == _code("BIWKV_ERR_SHAPE")
    assert _qs(L, out=K + 4) == _code("BIWKV_ERR_ALIAS")
    assert _qs(L, x=K + 2) == _code("BIWKV_ERR_ALIGN")
    assert _qs(L, x=None) == _code("BIWKV_ERR_NULL")
    assert _fused(L, dtype=3) == _code("BIWKV_ERR_DTYPE")


def test_valid_calls_report_missing_device(L):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a device is present; covered by the GPU tests")
    no_dev = _code("BIWKV_ERR_NO_DEVICE")
    assert _fwd(L) == no_dev
    assert _fused(L) == no_dev
    assert _qs(L) == no_dev
    flags = ctypes.c_uint32(7)
    assert L.biwkv_stream_fault_flags(None, ctypes.byref(flags)) == no_dev
    assert L.biwkv_stream_fault_flags(None, None) == _code("BIWKV_ERR_NULL")
    assert L.biwkv_release_scratch(None) == no_dev


def test_options_validate_and_report_previous(L):
    prev = ctypes.c_int64(-1)
    bad = _code("BIWKV_ERR_PARAM")
    assert L.biwkv_set_option(99, 1, None) == bad
    assert L.biwkv_set_option(_code("BIWKV_OPT_SPIN_LIMIT"), -1, None) == bad
    assert L.biwkv_set_option(_code("BIWKV_OPT_SPIN_LIMIT"), 2**32, None) == bad
    assert L.biwkv_set_option(_code("BIWKV_OPT_TWO_PASS"), 3, None) == bad
    assert L.biwkv_set_option(_code("BIWKV_OPT_WIDE_INDEX"), 2, None) == bad
    assert L.biwkv_set_option(_code("BIWKV_OPT_WIDE_INDEX"), -1, None) == bad
    # defaults, and the previous value comes back
    assert L.biwkv_set_option(_code("BIWKV_OPT_SPIN_LIMIT"), 7, ctypes.byref(prev)) == 0
    assert prev.value == 4096
    assert L.biwkv_set_option(_code("BIWKV_OPT_SPIN_LIMIT"), 4096, ctypes.byref(prev)) == 0
    assert prev.value == 7
    for name in ("BIWKV_OPT_TWO_PASS", "BIWKV_OPT_WIDE_INDEX"):
        assert L.biwkv_set_option(_code(name), 1, ctypes.byref(prev)) == 0
        assert prev.value == 0
        assert L.biwkv_set_option(_code(name), 0, ctypes.byref(prev)) == 0
        assert prev.value == 1
    assert L.biwkv_set_option(_code("BIWKV_OPT_XCD_LOCAL"), 2, None) == bad
    assert L.biwkv_set_option(_code("BIWKV_OPT_XCD_LOCAL"), 0, ctypes.byref(prev)) == 0
    assert prev.value == 1
    assert L.biwkv_set_option(_code("BIWKV_OPT_XCD_LOCAL"), 1, ctypes.byref(prev)) == 0
    assert prev.value == 0
    with lib.option(lib.OPT_TWO_PASS, 1):
        assert lib.set_option(lib.OPT_TWO_PASS, 1) == 1
    assert lib.set_option(lib.OPT_TWO_PASS, 0) == 0


def test_ceiling_library_exports_and_validates():
    """The measurement library (include/hbm_ceiling.h) loads, exports what its header declares,
    and rejects bad arguments before launching anything."""
    import os
    import re

    from linear_complexity_vision_amd import build

    if not os.path.exists(build.CEILING_LIB):
        pytest.skip("libhbmceiling.so is not built")
    C = ctypes.CDLL(build.CEILING_LIB)
    header = open(os.path.join(build.INCLUDE, "hbm_ceiling.h")).read()
    names = re.findall(r"^\s*\w+\s+(\w+)\s*\(", header, flags=re.M)
    assert names == ["hbm_stream"]
    for n in names:
        assert hasattr(C, n)
    f = C.hbm_stream
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    f.restype = ctypes.c_int
    K16, V16, O16 = 0x10000000, 0x20000000, 0x30000000
    assert f(K16, V16, O16, 0, 1, 0, 0, 1, 3, None) == 0            # empty: nothing launched
    assert f(K16, V16, O16, 64, 5, 0, 0, 1, 3, None) == -1          # dtype
    assert f(K16, V16, O16, 64, 1, 3, 0, 1, 3, None) == -1          # mode
    assert f(K16, V16, O16, 64, 1, 0, 0, 3, 3, None) == -1          # unroll
    assert f(K16, V16, O16, 64, 1, 0, 0, 1, 8, None) == -1          # policy
    assert f(K16, V16, O16, 12, 1, 0, 0, 1, 3, None) == -1          # not whole 16-byte pieces
    assert f(K16, V16, O16, 6, 1, 0, 0, 1, 7, None) == -1           # not whole 8-byte pieces
    assert f(K16, V16, O16, 5, 0, 0, 0, 1, 7, None) == -1           # fp32: not whole 8-byte pieces
    assert f(K16 + 4, V16, O16, 64, 1, 0, 0, 1, 3, None) == -1      # misaligned
    assert f(None, V16, O16, 64, 1, 0, 0, 1, 3, None) == -1         # NULL


def test_torch_front_end_refuses_host_tensors():
    import torch

    k = torch.zeros(1, 4, 2)
    w = torch.zeros(2)
    with pytest.raises(ValueError):
        lib.biwkv_forward(k, k, w, w)
    with pytest.raises(ValueError):
        lib.qshift(k, 2, 2)


def test_causal_forward_validation(L):
    def causal(k=K, v=V, w=WP, u=UP, out=OUT, B=2, T=8, C=4, dtype=lib.F32):
        return L.biwkv_causal_forward(k, v, w, u, out, B, T, C, dtype, None)

    assert causal(dtype=5) == _code("BIWKV_ERR_DTYPE")
    assert causal(v=None) == _code("BIWKV_ERR_NULL")
    assert causal(T=-1) == _code("BIWKV_ERR_SHAPE")
    assert causal(k=K + 2) == _code("BIWKV_ERR_ALIGN")
    assert causal(out=V + 4) == _code("BIWKV_ERR_ALIAS")
    assert causal(B=0) == 0


def test_qshift_mix_validation(L):
    def mix(x=K, mu=WP, out=OUT, B=1, H=2, W=4, C=4, n_mix=3, shift=1, gamma=0.25):
        return L.qshift_mix(x, mu, out, B, H, W, C, n_mix, shift, gamma, None)

    assert mix(n_mix=9) == _code("BIWKV_ERR_SHAPE")
    assert mix(n_mix=-1) == _code("BIWKV_ERR_SHAPE")
    assert mix(mu=None) == _code("BIWKV_ERR_NULL")
    assert mix(gamma=0.5) == _code("BIWKV_ERR_PARAM")
    assert mix(out=K + 64) == _code("BIWKV_ERR_ALIAS")
    assert mix(mu=OUT + 4 * 8) == _code("BIWKV_ERR_ALIAS")
    assert mix(x=K + 2) == _code("BIWKV_ERR_ALIGN")
    assert mix(n_mix=0, mu=None, out=None) == 0


def test_gated_forward_validation(L):
    R = 0x50000000

    def gated(k=K, v=V, r=R, w=WP, u=UP, out=OUT, B=2, T=8, C=4, dtype=lib.F32):
        return L.biwkv_gated_forward(k, v, r, w, u, out, B, T, C, dtype, None)

    assert gated(r=None) == _code("BIWKV_ERR_NULL")
    assert gated(r=R + 2) == _code("BIWKV_ERR_ALIGN")
    assert gated(r=R + 1, dtype=lib.BF16) == _code("BIWKV_ERR_ALIGN")
    assert gated(out=R) == _code("BIWKV_ERR_ALIAS")
    assert gated(dtype=9) == _code("BIWKV_ERR_DTYPE")
    assert gated(B=0, r=None) == 0


def test_backward_validation(L):
    G, DK, DV, DW, DU = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0x90001000

    def bwd(k=K, v=V, w=WP, u=UP, g=G, dk=DK, dv=DV, dw=DW, du=DU, B=2, T=8, C=4, dtype=lib.F32):
        return L.biwkv_backward(k, v, w, u, g, dk, dv, dw, du, B, T, C, dtype, None)

    assert bwd(dtype=4) == _code("BIWKV_ERR_DTYPE")
    assert bwd(g=None) == _code("BIWKV_ERR_NULL")
    assert bwd(dw=None) == _code("BIWKV_ERR_NULL")
    assert bwd(dk=DK + 2) == _code("BIWKV_ERR_ALIGN")
    assert bwd(dv=DK + 16) == _code("BIWKV_ERR_ALIAS")
    assert bwd(dk=G) == _code("BIWKV_ERR_ALIAS")
    assert bwd(du=DW + 8) == _code("BIWKV_ERR_ALIAS")
    assert bwd(T=-1) == _code("BIWKV_ERR_SHAPE")
    assert bwd(C=0, w=None, u=None, dw=None, du=None) == 0


def test_bidir_validation(L):
    def qb(x=K, out=OUT, B=1, N=8, C=4, shift=1, gamma=0.25):
        return L.qshift_bidir(x, out, B, N, C, shift, gamma, None)

    def fb(k=K, v=V, w=WP, u=UP, out=OUT, B=1, N=8, C=4, shift=1, gamma=0.25, dtype=lib.BF16):
        return L.biwkv_qshift_bidir_forward(k, v, w, u, out, B, N, C, shift, gamma, dtype, None)

    bad = _code("BIWKV_ERR_PARAM")
    for shift, gamma in [(1, 0.3), (1, -0.1), (1, math.nan), (-1, 0.25), (9, 0.25)]:
        assert qb(shift=shift, gamma=gamma) == bad, (shift, gamma)
        assert fb(shift=shift, gamma=gamma) == bad, (shift, gamma)
    # a shift of several tokens is valid on a sequence (a 1 x N grid would refuse it)
    assert _qs(L, H=1, W=8, shift=3) == bad
    assert qb(x=None) == _code("BIWKV_ERR_NULL")
    assert qb(N=-2) == _code("BIWKV_ERR_SHAPE")
    assert qb(x=K + 2) == _code("BIWKV_ERR_ALIGN")
    assert qb(out=K + 4) == _code("BIWKV_ERR_ALIAS")
    assert fb(dtype=9) == _code("BIWKV_ERR_DTYPE")
    assert fb(out=V + 4) == _code("BIWKV_ERR_ALIAS")
    assert qb(B=0, x=None, out=None) == 0
    assert fb(N=0, shift=0) == 0
    import torch

    if not torch.cuda.is_available():
        no_dev = _code("BIWKV_ERR_NO_DEVICE")
        assert qb(shift=3) == no_dev
        assert fb(shift=8) == no_dev


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        lib.load_library(str(tmp_path / "libbiwkv.so"))


def test_package_never_reaches_the_oracle():
    """The product path is the HIP library only: no module of the package imports the oracle or
    computes with numpy, and the library's sources include nothing from oracle/."""
    import os
    import re

    pkg = os.path.dirname(lib.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            path = os.path.join(root, f)
            if f.endswith(".py"):
                text = open(path).read()
                assert not re.search(r"^\s*(import|from)\s+(oracle|numpy)\b", text, flags=re.M), path
            elif f.endswith((".hip", ".h", ".cpp")):
                assert "oracle" not in open(path).read().lower(), path
