"""ctypes declarations of the C ABI in include/vdit_attn.h."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvdit_attn.so")

VDIT_OK = 0
STATUS_NAMES = {
    0: "VDIT_OK", 1: "VDIT_ERR_INVALID_ARG", 2: "VDIT_ERR_UNSUPPORTED", 3: "VDIT_ERR_ALIGNMENT",
    4: "VDIT_ERR_OUT_OF_MEMORY", 5: "VDIT_ERR_DEVICE", 6: "VDIT_ERR_WORKSPACE",
}
LAYOUT_NHD, LAYOUT_N3HD = 0, 1


class Desc(ctypes.Structure):
    """Mirror of vdit_attn_desc_t."""
    _fields_ = [
        ("nq", ctypes.c_int32), ("nk", ctypes.c_int32), ("heads_total", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("layout", ctypes.c_int32), ("head_begin", ctypes.c_int32),
        ("head_count", ctypes.c_int32), ("scale", ctypes.c_float), ("use_key_mask", ctypes.c_int32),
        ("use_rope", ctypes.c_int32), ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32), ("rope_dim_t", ctypes.c_int32), ("rope_dim_h", ctypes.c_int32),
        ("rope_dim_w", ctypes.c_int32), ("rope_base", ctypes.c_double), ("batch", ctypes.c_int32),
        ("qk_int8", ctypes.c_int32), ("vsa_cubes", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_ST = ctypes.c_int

# name -> (restype, argtypes); the order of this table follows the header
SIGNATURES = {
    "vdit_attn_ulysses_heads": (_ST, [_I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "vdit_attn_create": (_ST, [ctypes.POINTER(Desc), ctypes.POINTER(_P)]),
    "vdit_attn_destroy": (_ST, [_P]),
    "vdit_attn_workspace_bytes": (_ST, [_P, ctypes.POINTER(_S)]),
    "vdit_attn_fwd": (_ST, [_P, _P, _P, _P, _I, _P, _P, _S, _P]),
    "vdit_attn_prepare": (_ST, [_P, _P, _P, _P, _I, _P, _S, _P]),
    "vdit_attn_attend": (_ST, [_P, _P, _P, _P, _I, _P, _P, _S, _P]),
    "vdit_attn_fwd_noalloc": (_ST, [_P, _P, _P, _P, _I, _P, _P]),
    "vdit_attn_fwd_lens": (_ST, [_P, _P, _P, _P, ctypes.POINTER(_I), _P, _P, _S, _P]),
    "vdit_attn_prepare_lens": (_ST, [_P, _P, _P, _P, ctypes.POINTER(_I), _P, _S, _P]),
    "vdit_attn_attend_lens": (_ST, [_P, _P, _P, _P, ctypes.POINTER(_I), _P, _P, _S, _P]),
    "vdit_pack_heads": (_ST, [_P, _P, _I, _I, _I, _I, _P]),
    "vdit_unpack_heads": (_ST, [_P, _P, _I, _I, _I, _I, _P]),
    "vdit_attn_rope_probe": (_ST, [_P, _P, _P]),
    "vdit_vsa_keep": (_ST, [_P, ctypes.c_double, ctypes.POINTER(_I)]),
    "vdit_vsa_workspace_bytes": (_ST, [_P, _I, ctypes.POINTER(_S)]),
    "vdit_vsa_select": (_ST, [_P, _P, _P, _I, _P, _P, _S, _P]),
    "vdit_vsa_attend": (_ST, [_P, _P, _P, _P, _I, _P, _P, _P, _S, _P]),
    "vdit_vsa_fwd": (_ST, [_P, _P, _P, _P, _I, _P, _P, _S, _P]),
    "vdit_status_string": (ctypes.c_char_p, [_ST]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} is missing: build it with "
                "`python -c 'import __graft_entry__; __graft_entry__.build()'` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
