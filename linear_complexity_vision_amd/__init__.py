"""Vision-RWKV spatial-mix hot path (Bi-WKV and Q-Shift) for AMD Instinct MI355X.

The computation lives in libbiwkv.so (hand-written HIP for gfx950, C ABI in include/biwkv.h);
this package only marshals torch tensors to it.
"""
from ._lib import (  # noqa: F401
    BF16,
    F32,
    LIB_PATH,
    OPT_SPIN_LIMIT,
    OPT_TWO_PASS,
    OPT_WIDE_INDEX,
    OPT_XCD_LOCAL,
    BiwkvError,
    biwkv_backward,
    biwkv_causal_forward,
    biwkv_forward,
    biwkv_gated_forward,
    biwkv_qshift_bidir_forward,
    biwkv_qshift_forward,
    header_symbols,
    load_library,
    option,
    qshift,
    qshift_bidir,
    qshift_mix,
    release_scratch,
    set_option,
    status_codes,
    status_string,
    stream_fault_flags,
)
