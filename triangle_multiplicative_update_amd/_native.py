"""ctypes binding of ``libtrimul.so`` (the C ABI declared in ``include/trimul.h``).

Argument marshalling only. The library must have been built (``build.py``); if
it is missing, importing this module raises -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

# torch first: its HIP runtime is then the one the library binds to (same soname),
# so torch's streams and allocations are valid handles for the library.
import torch  # noqa: F401

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtrimul.so")

TRIMUL_OK = 0
TRIMUL_E_INVALID = 1
TRIMUL_E_UNSUPPORTED = 2
TRIMUL_E_DEVICE = 3
TRIMUL_OUTGOING = 0
TRIMUL_INCOMING = 1

# Every exported function and its C signature (mirrors include/trimul.h).
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_TENSOR_ARGS = [_vp] * 14
SIGNATURES = {
    "trimul_version": (ctypes.c_char_p, []),
    "trimul_last_error": (ctypes.c_char_p, []),
    "trimul_n_pad": (_i, [_i]),
    "trimul_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "trimul_check_support": (_i, [_i, _i, _i, _i, _i, _i]),
    "trimul_validate": (_i, _TENSOR_ARGS + [_i, _i, _i, _i, _i, _f, _vp, _vp, _sz]),
    "trimul_forward": (_i, _TENSOR_ARGS + [_i, _i, _i, _i, _i, _f, _vp, _vp, _sz, _vp]),
    "trimul_forward_stage": (_i, [_i] + _TENSOR_ARGS + [_i, _i, _i, _i, _i, _f, _vp, _vp, _sz, _vp]),
    "trimul_forward_noalloc": (_i, _TENSOR_ARGS + [_i, _i, _i, _i, _i, _f, _vp, _vp]),
    "trimul_graph_create": (_i, _TENSOR_ARGS + [_i, _i, _i, _i, _i, _f, _vp, _vp, _sz,
                                                ctypes.POINTER(_vp)]),
    "trimul_graph_launch": (_i, [_vp, _vp]),
    "trimul_graph_destroy": (_i, [_vp]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the gfx950 library first "
            "(python triangle_multiplicative_update_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def last_error() -> str:
    return lib.trimul_last_error().decode()


def version() -> str:
    return lib.trimul_version().decode()
