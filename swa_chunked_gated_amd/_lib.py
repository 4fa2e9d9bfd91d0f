"""ctypes loader of the in-tree HIP library ``libgdn_hybrid.so``.

There is no fallback: if the library is missing or fails to load, every call
raises, naming the build command.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn_hybrid.so")

_c_int = ctypes.c_int
_ptr = ctypes.c_void_p

# (name, restype, argtypes) of every symbol declared in include/gdn_hybrid.h
SIGNATURES = {
    "gdn_hybrid_version": (_c_int, []),
    "gdn_hybrid_strerror": (ctypes.c_char_p, [_c_int]),
    "gdn_hybrid_last_hip_error": (_c_int, []),
    "gdn_hybrid_set_test_faults": (_c_int, [_c_int, _c_int]),
    "gdn_hybrid_prefill_workspace": (
        _c_int, [_c_int] * 11 + [ctypes.POINTER(ctypes.c_size_t)]),
    "gdn_hybrid_prefill": (
        _c_int, [_ptr] * 7 + [_c_int] * 11 + [_ptr, ctypes.c_size_t, _ptr]),
    "gdn_hybrid_decode": (
        _c_int, [_ptr] * 12 + [_c_int] * 10 + [_ptr]),
    "gdn_hybrid_prefill_weighted": (
        _c_int, [_ptr] * 7 + [_c_int] * 11 + [ctypes.c_float] * 2 + [_ptr, ctypes.c_size_t, _ptr]),
    "gdn_hybrid_prefill_noalloc": (
        _c_int, [_ptr] * 7 + [_c_int] * 11 + [_ptr]),
    "gdn_hybrid_noalloc_max_workspace": (ctypes.c_size_t, []),
    "gdn_hybrid_prefill_backward_workspace": (
        _c_int, [_c_int] * 10 + [ctypes.POINTER(ctypes.c_size_t)]),
    "gdn_hybrid_prefill_backward": (
        _c_int, [_ptr] * 12 + [_c_int] * 10 + [ctypes.c_float] * 2 + [_ptr, ctypes.c_size_t, _ptr]),
    "gdn_hybrid_decode_weighted": (
        _c_int, [_ptr] * 12 + [_c_int] * 10 + [ctypes.c_float] * 2 + [_ptr]),
    "gdn_hybrid_cache_from_prefill": (
        _c_int, [_ptr] * 8 + [_c_int] * 10 + [_ptr]),
    "shortconv_qkv": (
        _c_int, [_ptr] * 9 + [_c_int] * 6 + [ctypes.c_float, _c_int, _c_int, _c_int, _ptr]),
    "shortconv_history_from_prefill": (
        _c_int, [_ptr] * 6 + [_c_int] * 6 + [ctypes.c_float, _c_int, _c_int, _c_int, _ptr]),
    "shortconv_qkv_decode": (
        _c_int, [_ptr] * 13 + [_c_int] * 5 + [ctypes.c_float, _c_int, _c_int, _c_int, _ptr]),
}

_lib = None


class GdnError(RuntimeError):
    """A library call returned a negative status code."""

    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (code {code})")
        self.code = code


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m swa_chunked_gated_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, code: int) -> None:
    if code != 0:
        lib = load()
        msg = lib.gdn_hybrid_strerror(code).decode()
        if code == -4:
            msg += f" (hipError {lib.gdn_hybrid_last_hip_error()})"
        raise GdnError(fn, code, msg)
