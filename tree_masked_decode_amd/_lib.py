"""ctypes binding of libtreeattn.so (the C ABI in include/tree_attn.h).

Argument marshalling only: every step of the path runs in the HIP library.
The library must be built (``python -m tree_masked_decode_amd.build``); a
missing library is an error, never a fallback.

torch is imported before the library is opened so that both share torch's
HIP runtime (libamdhip64.so.7 is then already loaded and is reused).
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  -- must precede loading the HIP library

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtreeattn.so")

TA_OK = 0
TA_EINVAL = -1
TA_ESIZE = -2
TA_EOVERFLOW = -3
TA_EUNSUPPORTED = -4
TA_EHIP = -5
TA_F32 = 0
TA_F16 = 1
TA_BF16 = 2
TA_MASK_NONE = 0
TA_MASK_F16 = 1
TA_MASK_BOOL = 2

EXPORTS = (
    "tree_attn_partials_bytes",
    "tree_attn_pick_nwg",
    "tree_attn_quant_pick_nwg",
    "tree_attn_quant_pick_nwg_ex",
    "tree_attn_forward",
    "tree_attn_decode",
    "tree_attn_reduce",
    "tree_attn_forward_noalloc",
    "tree_attn_quant_forward",
    "tree_attn_quant_forward_ex",
    "build_tree_mask",
    "tree_attn_last_error",
)

_lock = threading.Lock()
_lib = None


class LibraryMissing(RuntimeError):
    pass


def load():
    """Open libtreeattn.so and declare every exported signature."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                "libtreeattn.so is not built (%s); run "
                "`python -m tree_masked_decode_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        U = ctypes.c_uint32
        Z = ctypes.c_size_t
        I = ctypes.c_int
        F = ctypes.c_float
        lib.tree_attn_partials_bytes.argtypes = [U, U, U, U]
        lib.tree_attn_partials_bytes.restype = Z
        lib.tree_attn_pick_nwg.argtypes = [U, U, U, U, U, I, U]
        lib.tree_attn_pick_nwg.restype = U
        lib.tree_attn_quant_pick_nwg.argtypes = [U, U, U, U, U, U, U]
        lib.tree_attn_quant_pick_nwg.restype = U
        lib.tree_attn_quant_pick_nwg_ex.argtypes = [U, U, U, U, U, U, U, U, I, I, U]
        lib.tree_attn_quant_pick_nwg_ex.restype = U
        lib.tree_attn_forward.argtypes = [P, Z, P, P, I, Z, P, Z, P, Z, P, Z,
                                          U, U, U, U, U, U, U, F, U, P]
        lib.tree_attn_forward.restype = I
        lib.tree_attn_decode.argtypes = [P, Z, P, P, I, Z, P, Z, P, Z,
                                         U, U, U, U, U, U, U, F, U, P]
        lib.tree_attn_decode.restype = I
        lib.tree_attn_reduce.argtypes = [P, Z, P, I, Z, U, U, U, P]
        lib.tree_attn_reduce.restype = I
        lib.tree_attn_forward_noalloc.argtypes = [P, Z, P, P, I, Z, P, Z, P, Z,
                                                  U, U, U, U, U, U, U, F, U, P]
        lib.tree_attn_forward_noalloc.restype = I
        lib.tree_attn_quant_forward.argtypes = [
            P, I, Z, P, P, P, P, P, P, ctypes.POINTER(Z), P, Z, P, Z,
            ctypes.c_uint64, U, P, Z, P, Z, U, U, U, U, U, U, U, U, U, F, U, P]
        lib.tree_attn_quant_forward.restype = I
        lib.tree_attn_quant_forward_ex.argtypes = [
            P, I, Z, P, P, P, P, P, P, ctypes.POINTER(Z), P, Z, P, I, Z,
            ctypes.c_uint64, U, U, P, Z, P, Z, U, U, U, U, U, U, U, U, U, F, U, P]
        lib.tree_attn_quant_forward_ex.restype = I
        lib.build_tree_mask.argtypes = [P, U, U, U, P, Z, P]
        lib.build_tree_mask.restype = I
        lib.tree_attn_last_error.argtypes = []
        lib.tree_attn_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def last_error() -> str:
    return load().tree_attn_last_error().decode()
