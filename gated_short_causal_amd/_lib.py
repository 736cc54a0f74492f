"""ctypes loader for liblfm2sc.so (the C ABI declared in include/lfm2sc.h).

torch is imported first so that the HIP runtime torch ships with is the one
the library binds to (both name it by the same soname).  A missing library is
an error, never a fallback.
"""
import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime before the library)

_PKG = os.path.dirname(os.path.abspath(__file__))
# LFM2SC_LIB may name another build of the same library (e.g. a tuning variant) to load instead.
LIB_PATH = os.environ.get("LFM2SC_LIB") or os.path.join(_PKG, "liblfm2sc.so")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_size = ctypes.c_size_t

# (name, restype, argtypes) for every symbol of include/lfm2sc.h
SIGNATURES = {
    "lfm2sc_prefill_ragged": (_int, [_int, _int, _int, _vp, _i64, _i64, _vp, _int, _vp, _vp, _vp, _i64, _i64, _vp,
                                     _vp, _i64, _vp]),
    "lfm2sc_decode_step": (_int, [_int, _int, _int, _vp, _i64, _int, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp]),
    "lfm2sc_verify_window": (_int, [_int, _int, _int, _vp, _i64, _int, _int, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp,
                                    _i64, _vp]),
    "lfm2sc_commit_window": (_int, [_int, _int, _int, _vp, _int, _int, _vp, _vp, _i64, _i64, _vp, _vp]),
    "lfm2sc_backward_workspace_bytes": (_size, [_int, _int, _int, _i64, _int]),
    "lfm2sc_backward": (_int, [_int, _int, _int, _vp, _i64, _i64, _vp, _int, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64,
                               _vp, _vp, _i64, _vp, _vp, _vp, _vp, _size, _vp]),
    "lfm2sc_backward_noalloc": (_int, [_int, _int, _int, _vp, _i64, _i64, _vp, _int, _vp, _vp, _vp, _i64, _i64, _vp,
                                       _vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _vp]),
    "lfm2sc_fused_prefill_workspace_bytes": (_size, [_int, _int, _int, _int, _int]),
    "lfm2sc_fused_prefill_plan": (_int, [_int, _int, _int, _i64]),
    "lfm2sc_fused_prefill": (_int, [_int, _int, _int, _int, _vp, _i64, _i64, _vp, _int, _vp, _vp, _vp, _vp, _i64, _i64,
                                    _vp, _vp, _i64, _vp, _i64, _vp, _size, _vp]),
    "lfm2sc_conv_update": (_int, [_int, _int, _int, _int, _int, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _vp,
                                  _vp, _vp, _i64, _i64, _i64, _vp]),
    "lfm2sc_status_string": (ctypes.c_char_p, [_int]),
    "lfm2sc_last_error": (ctypes.c_char_p, []),
    "lfm2sc_abi_version": (_int, []),
}

_lib = None


def lib():
    """The loaded library with argument types set; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"liblfm2sc.so not found at {LIB_PATH}: build it with `python -m gated_short_causal_amd.build` "
            "(there is no fallback implementation)")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    _lib = handle
    return handle
