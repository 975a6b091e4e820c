"""MI355X-native attention for video diffusion transformers (one device's head share).

The computation lives in the HIP library ``libvdit_attn.so`` (C ABI in
``include/vdit_attn.h``); this package is a thin ctypes binding over it.
"""
from .api import (  # noqa: F401
    Attention,
    VditError,
    pack_heads,
    unpack_heads,
    status_string,
    ulysses_heads,
    make_desc,
    create_raw,
)
from ._lib import LIB_PATH, load as load_library  # noqa: F401
