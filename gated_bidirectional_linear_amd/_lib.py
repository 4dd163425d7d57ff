"""Loading of the in-tree HIP library and its ctypes signatures.

The library is the product: there is no fallback.  If ``libgla.so`` is absent
or does not load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgla.so")

# Exported symbols and their ctypes signatures, in the order include/gla.h
# declares them.
_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
SIGNATURES = {
    "gla_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp, _i]),
    "gla_block_causal_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                      _vp, _vp, _i, _i]),
    "gla_block_causal_forward_at": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                         _vp, _vp, _i, _i, _i]),
    "gla_token_causal_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                      _vp, _vp, _i, _i, _i]),
    "gla_forward_batch": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i]),
    "gla_block_causal_forward_batch": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp,
                                            _vp, _vp, _vp, _i, _i, _i]),
    "gla_token_causal_forward_batch": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp,
                                            _vp, _vp, _vp, _i, _i, _i]),
    "gla_status_string": (ctypes.c_char_p, [_i]),
    "gla_version": (_i, []),
    "gla_timing_enable": (_i, [_i]),
    "gla_timing_read": (_i, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong), _i]),
    "gla_kernel_name": (ctypes.c_char_p, [_i]),
}

_LIB = None


class LibraryNotBuilt(RuntimeError):
    pass


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the HIP library; raise if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            f"{path} is missing: build it with `python -m gated_bidirectional_linear_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib
