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
# and then include/gla_internal.h declare them.
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
    "gla_forward_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp, _i]),
    "gla_status_string": (ctypes.c_char_p, [_i]),
    "gla_version": (_i, []),
    "gla_timing_enable": (_i, [_i]),
    "gla_timing_read": (_i, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong), _i]),
    "gla_kernel_name": (ctypes.c_char_p, [_i]),
    "gla_timing_select": (_i, [ctypes.c_uint]),
    "gla_plan_override": (_i, [_i, _i]),
    "gla_plan_describe": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(_i), _i]),
}

_LIB = None


class LibraryNotBuilt(RuntimeError):
    pass


def hip_runtimes() -> list:
    """Files of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the HIP library; raise if it is missing.

    The library must share the HIP runtime of the process's PyTorch, which
    owns the device memory and streams it is handed.  PyTorch ships its own
    copy of the runtime; importing it first lets the dynamic linker satisfy
    the library's runtime dependency with that copy.  Loaded the other way
    round, a second runtime (with its own HSA runtime) would come in beside
    it, and PyTorch's streams would be foreign to the library.  A process
    that already holds two runtimes is refused."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            f"{path} is missing: build it with `python -m gated_bidirectional_linear_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    import torch  # noqa: F401  (binds the library to PyTorch's HIP runtime)
    lib = ctypes.CDLL(path)
    runtimes = hip_runtimes()
    if len(runtimes) > 1:
        raise RuntimeError("more than one HIP runtime is loaded in this process (" + ", ".join(runtimes) +
                           "): load PyTorch before any other HIP library")
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib
