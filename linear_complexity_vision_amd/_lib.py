"""ctypes binding of libbiwkv.so: argument marshalling only.

Every step of the computation runs in the HIP library; this module checks tensor metadata,
allocates outputs with torch, passes raw device pointers and torch's current HIP stream, and turns
status codes into exceptions. There is no fallback: if the library is missing, calls fail.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbiwkv.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "biwkv.h")

F32 = 0
BF16 = 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_lib = None


class BiwkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libbiwkv status {status}: {message}")
        self.status = status


def header_symbols() -> list[str]:
    """Names of the functions declared in include/biwkv.h."""
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)


def status_codes() -> dict[str, int]:
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(BIWKV_\w+)\s+\(?(-?\d+)\)?", text)}


def load_library(path: str | None = None) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libbiwkv.so is not built ({p}); run __graft_entry__.build() first")
    # torch (which supplies device memory and streams) loads its HIP runtime first, so the library
    # binds to that same runtime instead of bringing a second one into the process
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    lib.biwkv_forward.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P]
    lib.biwkv_forward.restype = ctypes.c_int
    lib.biwkv_forward_noalloc.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P]
    lib.biwkv_forward_noalloc.restype = ctypes.c_int
    lib.biwkv_causal_forward.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P]
    lib.biwkv_causal_forward.restype = ctypes.c_int
    lib.biwkv_backward.argtypes = [_P] * 9 + [_I64, _I64, _I64, ctypes.c_int, _P]
    lib.biwkv_backward.restype = ctypes.c_int
    lib.biwkv_gated_forward.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P]
    lib.biwkv_gated_forward.restype = ctypes.c_int
    lib.qshift.argtypes = [_P, _P, _I64, _I64, _I64, _I64, ctypes.c_int, ctypes.c_double, _P]
    lib.qshift.restype = ctypes.c_int
    lib.qshift_mix.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_int, ctypes.c_int,
                               ctypes.c_double, _P]
    lib.qshift_mix.restype = ctypes.c_int
    lib.biwkv_qshift_forward.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_int,
                                         ctypes.c_double, ctypes.c_int, _P]
    lib.biwkv_qshift_forward.restype = ctypes.c_int
    lib.qshift_bidir.argtypes = [_P, _P, _I64, _I64, _I64, ctypes.c_int, ctypes.c_double, _P]
    lib.qshift_bidir.restype = ctypes.c_int
    lib.biwkv_qshift_bidir_forward.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_int,
                                               ctypes.c_double, ctypes.c_int, _P]
    lib.biwkv_qshift_bidir_forward.restype = ctypes.c_int
    lib.biwkv_status_string.argtypes = [ctypes.c_int]
    lib.biwkv_status_string.restype = ctypes.c_char_p
    lib.biwkv_last_hip_error.argtypes = []
    lib.biwkv_last_hip_error.restype = ctypes.c_int
    lib.biwkv_stream_fault_flags.argtypes = [_P, ctypes.POINTER(ctypes.c_uint32)]
    lib.biwkv_stream_fault_flags.restype = ctypes.c_int
    lib.biwkv_version.argtypes = []
    lib.biwkv_version.restype = ctypes.c_int
    lib.biwkv_release_scratch.argtypes = [_P]
    lib.biwkv_release_scratch.restype = ctypes.c_int
    lib.biwkv_set_option.argtypes = [ctypes.c_int, _I64, ctypes.POINTER(_I64)]
    lib.biwkv_set_option.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().biwkv_status_string(int(status)).decode()


def _check(rc: int) -> None:
    if rc != 0:
        lib = load_library()
        msg = lib.biwkv_status_string(rc).decode()
        if rc == -8:
            msg += f" (hipError_t {lib.biwkv_last_hip_error()})"
        raise BiwkvError(rc, msg)


# ------------------------------------------------------------------------------------------
# torch-tensor front end (torch is used for device memory and the current stream only)
# ------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _kv_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"k and v must be float32 or bfloat16, got {t.dtype}")


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_bitc(k, v, w, u):
    torch = _torch()
    _require(k.is_cuda and v.is_cuda and w.is_cuda and u.is_cuda, "all tensors must be on a HIP device")
    _require(k.dim() == 3 and v.shape == k.shape, "k and v must both be [B, T, C]")
    _require(k.dtype == v.dtype, "k and v must share a dtype")
    _require(w.dtype == torch.float32 and u.dtype == torch.float32, "w and u must be float32")
    _require(w.dim() == 1 and u.dim() == 1 and w.numel() == k.shape[2] and u.numel() == k.shape[2],
             "w and u must be [C]")
    for t in (k, v, w, u):
        _require(t.is_contiguous(), "all tensors must be contiguous")
    return _kv_dtype(k)


def biwkv_forward(k, v, w, u, out=None):
    """Bi-WKV forward (Eq. (5)); k, v: [B, T, C] float32 or bfloat16, w, u: [C] float32 -> float32."""
    torch = _torch()
    dt = _check_bitc(k, v, w, u)
    B, T, C = k.shape
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=k.device)
    _require(out.shape == k.shape and out.dtype == torch.float32 and out.is_contiguous(),
             "out must be a contiguous float32 [B, T, C] tensor")
    with torch.cuda.device(k.device):
        _check(load_library().biwkv_forward(k.data_ptr(), v.data_ptr(), w.data_ptr(), u.data_ptr(),
                                            out.data_ptr(), B, T, C, dt, _stream_handle(k.device)))
    return out


def biwkv_backward(k, v, w, u, g):
    """Gradients of a loss through biwkv_forward(k, v, w, u) given g = dL/dy (float32 [B, T, C]):
    returns dk, dv (float32 [B, T, C]) and dw, du (float32 [C], summed over the batch)."""
    torch = _torch()
    dt = _check_bitc(k, v, w, u)
    _require(g.is_cuda and g.shape == k.shape and g.dtype == torch.float32 and g.is_contiguous(),
             "g must be a contiguous float32 tensor shaped like k")
    B, T, C = k.shape
    dk = torch.empty((B, T, C), dtype=torch.float32, device=k.device)
    dv = torch.empty_like(dk)
    dw = torch.empty((C,), dtype=torch.float32, device=k.device)
    du = torch.empty_like(dw)
    with torch.cuda.device(k.device):
        _check(load_library().biwkv_backward(k.data_ptr(), v.data_ptr(), w.data_ptr(), u.data_ptr(),
                                             g.data_ptr(), dk.data_ptr(), dv.data_ptr(), dw.data_ptr(),
                                             du.data_ptr(), B, T, C, dt, _stream_handle(k.device)))
    return dk, dv, dw, du


def biwkv_causal_forward(k, v, w, u, out=None):
    """Causal attention (Eq. (7) with b = d = 0: earlier tokens plus the bonus term); same
    arguments and exponent convention as biwkv_forward."""
    torch = _torch()
    dt = _check_bitc(k, v, w, u)
    B, T, C = k.shape
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=k.device)
    _require(out.shape == k.shape and out.dtype == torch.float32 and out.is_contiguous(),
             "out must be a contiguous float32 [B, T, C] tensor")
    with torch.cuda.device(k.device):
        _check(load_library().biwkv_causal_forward(k.data_ptr(), v.data_ptr(), w.data_ptr(),
                                                   u.data_ptr(), out.data_ptr(), B, T, C, dt,
                                                   _stream_handle(k.device)))
    return out


def biwkv_gated_forward(k, v, r, w, u, out=None):
    """Eq. (2) before the output projection: sigmoid(r) * Bi-WKV(k, v); r like k (same dtype)."""
    torch = _torch()
    dt = _check_bitc(k, v, w, u)
    _require(r.is_cuda and r.shape == k.shape and r.dtype == k.dtype and r.is_contiguous(),
             "r must be a contiguous tensor shaped and typed like k")
    B, T, C = k.shape
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=k.device)
    _require(out.shape == k.shape and out.dtype == torch.float32 and out.is_contiguous(),
             "out must be a contiguous float32 [B, T, C] tensor")
    with torch.cuda.device(k.device):
        _check(load_library().biwkv_gated_forward(k.data_ptr(), v.data_ptr(), r.data_ptr(), w.data_ptr(),
                                                  u.data_ptr(), out.data_ptr(), B, T, C, dt,
                                                  _stream_handle(k.device)))
    return out


def biwkv_qshift_forward(k, v, w, u, H, W, shift=1, gamma=0.25, out=None):
    """Fused Bi-WKV(Q-Shift(k), Q-Shift(v)) on an H x W token grid (T = H * W)."""
    torch = _torch()
    dt = _check_bitc(k, v, w, u)
    B, T, C = k.shape
    _require(T == H * W, "T must equal H * W")
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=k.device)
    _require(out.shape == k.shape and out.dtype == torch.float32 and out.is_contiguous(),
             "out must be a contiguous float32 [B, T, C] tensor")
    with torch.cuda.device(k.device):
        _check(load_library().biwkv_qshift_forward(
            k.data_ptr(), v.data_ptr(), w.data_ptr(), u.data_ptr(), out.data_ptr(), B, H, W, C,
            int(shift), float(gamma), dt, _stream_handle(k.device)))
    return out


def qshift(x, H, W, shift=1, gamma=0.25, out=None):
    """Q-Shift X-dagger of a [B, H*W, C] float32 tensor (bit-exact gather with zero fill)."""
    torch = _torch()
    _require(x.is_cuda and x.dtype == torch.float32 and x.dim() == 3 and x.is_contiguous(),
             "x must be a contiguous float32 [B, N, C] tensor on a HIP device")
    B, N, C = x.shape
    _require(N == H * W, "N must equal H * W")
    if out is None:
        out = torch.empty_like(x)
    _require(out.shape == x.shape and out.dtype == torch.float32 and out.is_contiguous(),
             "out must match x")
    with torch.cuda.device(x.device):
        _check(load_library().qshift(x.data_ptr(), out.data_ptr(), B, H, W, C, int(shift),
                                     float(gamma), _stream_handle(x.device)))
    return out


def qshift_bidir(x, shift=1, gamma=0.25, out=None):
    """Bidirectional shift of a [B, N, C] float32 token sequence (the MAE form of Q-Shift: the
    right/down groups take token n - shift, the left/up groups n + shift); bit-exact gather."""
    torch = _torch()
    _require(x.is_cuda and x.dtype == torch.float32 and x.dim() == 3 and x.is_contiguous(),
             "x must be a contiguous float32 [B, N, C] tensor on a HIP device")
    B, N, C = x.shape
    if out is None:
        out = torch.empty_like(x)
    _require(out.shape == x.shape and out.dtype == torch.float32 and out.is_contiguous(),
             "out must match x")
    with torch.cuda.device(x.device):
        _check(load_library().qshift_bidir(x.data_ptr(), out.data_ptr(), B, N, C, int(shift),
                                           float(gamma), _stream_handle(x.device)))
    return out


def biwkv_qshift_bidir_forward(k, v, w, u, shift=1, gamma=0.25, out=None):
    """Fused Bi-WKV(qshift_bidir(k), qshift_bidir(v)) over a sparse token sequence (T = N)."""
    torch = _torch()
    dt = _check_bitc(k, v, w, u)
    B, T, C = k.shape
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=k.device)
    _require(out.shape == k.shape and out.dtype == torch.float32 and out.is_contiguous(),
             "out must be a contiguous float32 [B, T, C] tensor")
    with torch.cuda.device(k.device):
        _check(load_library().biwkv_qshift_bidir_forward(
            k.data_ptr(), v.data_ptr(), w.data_ptr(), u.data_ptr(), out.data_ptr(), B, T, C,
            int(shift), float(gamma), dt, _stream_handle(k.device)))
    return out


def qshift_mix(x, mu, H, W, shift=1, gamma=0.25, out=None):
    """Eq. (9) mixing: out[j] = x + (1 - mu[j]) * X-dagger(x); x [B, H*W, C], mu [J, C] float32
    -> [J, B, H*W, C] float32."""
    torch = _torch()
    _require(x.is_cuda and mu.is_cuda, "x and mu must be on a HIP device")
    _require(x.dtype == torch.float32 and x.dim() == 3 and x.is_contiguous(),
             "x must be a contiguous float32 [B, N, C] tensor")
    B, N, C = x.shape
    _require(N == H * W, "N must equal H * W")
    _require(mu.dtype == torch.float32 and mu.dim() == 2 and mu.shape[1] == C and mu.is_contiguous(),
             "mu must be a contiguous float32 [J, C] tensor")
    J = mu.shape[0]
    if out is None:
        out = torch.empty((J, B, N, C), dtype=torch.float32, device=x.device)
    _require(out.shape == (J, B, N, C) and out.dtype == torch.float32 and out.is_contiguous(),
             "out must be a contiguous float32 [J, B, N, C] tensor")
    with torch.cuda.device(x.device):
        _check(load_library().qshift_mix(x.data_ptr(), mu.data_ptr(), out.data_ptr(), B, H, W, C, J,
                                         int(shift), float(gamma), _stream_handle(x.device)))
    return out


def stream_fault_flags(device=None) -> int:
    """Synchronises torch's current stream and returns (and clears) its scratch fault bits."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    flags = ctypes.c_uint32(0)
    with torch.cuda.device(dev):
        _check(load_library().biwkv_stream_fault_flags(_stream_handle(dev), ctypes.byref(flags)))
    return int(flags.value)


OPT_SPIN_LIMIT = 1
OPT_TWO_PASS = 2
OPT_WIDE_INDEX = 3
OPT_XCD_LOCAL = 4


def set_option(option: int, value: int) -> int:
    """Sets a process-wide library option (OPT_*); returns the previous value."""
    prev = _I64(0)
    _check(load_library().biwkv_set_option(int(option), int(value), ctypes.byref(prev)))
    return int(prev.value)


class option:
    """Context manager that sets a library option and restores its previous value."""

    def __init__(self, opt: int, value: int):
        self.opt, self.value, self.prev = opt, value, None

    def __enter__(self):
        self.prev = set_option(self.opt, self.value)
        return self

    def __exit__(self, *exc):
        set_option(self.opt, self.prev)
        return False


def release_scratch(device=None) -> None:
    """Releases the library's scratch for torch's current stream (stream-ordered free)."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        _check(load_library().biwkv_release_scratch(_stream_handle(dev)))
