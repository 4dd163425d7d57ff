"""Gated bidirectional ReLU linear attention on MI355X (gfx950).

Thin Python binding over the C ABI of ``libgla.so`` (declared in
``include/gla.h``).  It only checks tensors and marshals device pointers and
the current HIP stream; every step of the operator runs in the HIP kernels.
PyTorch provides device memory and streams.

    out = forward(q, k, v, beta, g, rms_w, (T, H, W), eps=1e-6)
    out = block_causal_forward(q, k, v, beta, g, rms_w, (T, H, W), state_S, state_z,
                               block_frames, eps=1e-6)
    out = token_causal_forward(q, k, v, beta, g, rms_w, (T, H, W), state_S, state_z,
                               include_self=True, eps=1e-6)

q, k, v, g: [N, heads, d] (float32, bfloat16, float8_e4m3fn or float8_e5m2,
contiguous, on the GPU),
beta: [N, heads] same dtype, rms_w: [d] float32, N = T*H*W, d in {32, 64, 128}.
A leading batch dimension ([B, N, heads, d], beta [B, N, heads], states
[B, heads, d, d] and [B, heads, d]) runs B independent sequences of the same
grid in one call.
"""
from __future__ import annotations

import ctypes

from ._lib import LIB_PATH, LibraryNotBuilt, SIGNATURES, load

__all__ = [
    "forward",
    "forward_noalloc",
    "block_causal_forward",
    "token_causal_forward",
    "status_string",
    "version",
    "GlaError",
    "LibraryNotBuilt",
    "LIB_PATH",
    "SIGNATURES",
    "timing_enable",
    "timing_read",
    "timing_select",
    "plan_override",
    "plan_reset",
    "plan_describe",
    "PLAN_FIELDS",
    "PLAN_KNOBS",
    "DTYPE_F32",
    "DTYPE_BF16",
    "DTYPE_FP8_E4M3",
    "DTYPE_FP8_E5M2",
]

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_FP8_E4M3 = 2
DTYPE_FP8_E5M2 = 3
NUM_KERNELS = 4


class GlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def status_string(status: int) -> str:
    return load().gla_status_string(int(status)).decode()


def version() -> int:
    return int(load().gla_version())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float8_e4m3fn:
        return DTYPE_FP8_E4M3
    if t.dtype == torch.float8_e5m2:
        return DTYPE_FP8_E5M2
    raise TypeError(f"unsupported dtype {t.dtype}; use float32, bfloat16, float8_e4m3fn or float8_e5m2")


def _check(name, t, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _common(q, k, v, beta, g, rms_w, grid, out):
    """Checks the tensors; returns (batch or None, T, H, W, heads, d, dtype code, out)."""
    torch = _torch()
    if q.dim() not in (3, 4):
        raise ValueError("q must be [N, heads, d] or [B, N, heads, d]")
    T, H, W = (int(x) for x in grid)
    batch = int(q.shape[0]) if q.dim() == 4 else None
    N, heads, d = (int(x) for x in q.shape[-3:])
    if N != T * H * W:
        raise ValueError(f"q has {N} tokens but the grid {T}x{H}x{W} has {T * H * W}")
    if batch is not None and batch < 1:
        raise ValueError("the batch dimension must be at least 1")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    dt = q.dtype
    code = _dtype_code(q)
    bshape = tuple(q.shape[:-1])
    for name, t, shp in (("k", k, q.shape), ("v", v, q.shape), ("g", g, q.shape), ("beta", beta, bshape),
                         ("q", q, q.shape)):
        _check(name, t, shp, dt, q.device)
    _check("rms_w", rms_w, (d,), torch.float32, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, q.shape, dt, q.device)
    return batch, T, H, W, heads, d, code, out


def _check_state(state_S, state_z, batch, heads, d, device):
    torch = _torch()
    lead = () if batch is None else (batch,)
    _check("state_S", state_S, lead + (heads, d, d), torch.float32, device)
    _check("state_z", state_z, lead + (heads, d), torch.float32, device)


def _stream_handle(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else ctypes.c_void_p(0)


def forward(q, k, v, beta, g, rms_w, grid, eps: float = 1e-6, out=None, stream=None):
    """Bidirectional operator; returns ``out`` (allocated if not given)."""
    batch, T, H, W, heads, d, code, out = _common(q, k, v, beta, g, rms_w, grid, out)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(rms_w))
    tail = (T, H, W, heads, d, float(eps), _ptr(out), _stream_handle(stream, q.device), code)
    if batch is None:
        st, where = load().gla_forward(*args, *tail), "gla_forward"
    else:
        st, where = load().gla_forward_batch(*args, batch, *tail), "gla_forward_batch"
    if st != 0:
        raise GlaError(st, where)
    return out


def forward_noalloc(q, k, v, beta, g, rms_w, grid, eps: float = 1e-6, out=None, stream=None):
    """The bidirectional operator through gla_forward_noalloc: the library
    allocates no device memory (its scratch is a static 64 MiB device array;
    calls that overlap on one device race on it).  ``out`` must be given by
    callers that cannot allocate; otherwise it is allocated here.  Returns
    ``out``."""
    batch, T, H, W, heads, d, code, out = _common(q, k, v, beta, g, rms_w, grid, out)
    if batch is not None:
        raise ValueError("forward_noalloc takes one sequence ([N, heads, d] tensors)")
    st = load().gla_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(rms_w), T, H, W, heads,
                                    d, float(eps), _ptr(out), _stream_handle(stream, q.device), code)
    if st != 0:
        raise GlaError(st, "gla_forward_noalloc")
    return out


def block_causal_forward(q, k, v, beta, g, rms_w, grid, state_S, state_z, block_frames: int,
                         eps: float = 1e-6, out=None, stream=None, t_offset: int = 0):
    """Block-causal operator.  ``state_S`` [heads, d, d] and ``state_z`` [heads, d]
    (float32) are read as the carried state and overwritten in place with the
    state after the last block.  ``t_offset`` is the absolute frame of the
    call's first frame (a multiple of ``block_frames``) when a long video is
    streamed through successive calls.  Returns ``out``."""
    batch, T, H, W, heads, d, code, out = _common(q, k, v, beta, g, rms_w, grid, out)
    _check_state(state_S, state_z, batch, heads, d, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(rms_w))
    tail = (T, H, W, heads, d, float(eps), _ptr(out), _stream_handle(stream, q.device), _ptr(state_S),
            _ptr(state_z), int(block_frames), int(t_offset), code)
    if batch is None:
        st, where = load().gla_block_causal_forward_at(*args, *tail), "gla_block_causal_forward_at"
    else:
        st, where = load().gla_block_causal_forward_batch(*args, batch, *tail), "gla_block_causal_forward_batch"
    if st != 0:
        raise GlaError(st, where)
    return out


def token_causal_forward(q, k, v, beta, g, rms_w, grid, state_S, state_z, include_self: bool = True,
                         eps: float = 1e-6, out=None, stream=None, t_offset: int = 0):
    """Token-level causal operator: token i reads the carried state plus the
    tokens j <= i (``include_self``) or j < i.  ``state_S`` [heads, d, d] and
    ``state_z`` [heads, d] (float32) are read and overwritten in place with the
    state after the last token.  ``t_offset`` is the absolute frame of the
    call's first frame when a sequence is streamed through successive calls.
    Returns ``out``."""
    batch, T, H, W, heads, d, code, out = _common(q, k, v, beta, g, rms_w, grid, out)
    _check_state(state_S, state_z, batch, heads, d, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(rms_w))
    tail = (T, H, W, heads, d, float(eps), _ptr(out), _stream_handle(stream, q.device), _ptr(state_S),
            _ptr(state_z), 1 if include_self else 0, int(t_offset), code)
    if batch is None:
        st, where = load().gla_token_causal_forward(*args, *tail), "gla_token_causal_forward"
    else:
        st, where = load().gla_token_causal_forward_batch(*args, batch, *tail), "gla_token_causal_forward_batch"
    if st != 0:
        raise GlaError(st, where)
    return out


# Launch-plan knobs of include/gla_internal.h (tests and tuning sweeps only).
PLAN_KNOBS = {
    "pass1_generic": 0,
    "pass1_workgroups": 1,
    "pass2_generic": 2,
    "pass2_workgroups": 3,
    "rope_global": 4,
    "token_causal_workgroups": 5,
    "pass2_heads": 6,
}


def plan_override(knob: str, value: int) -> None:
    """Set a launch-plan knob (0 = default).  Process-wide; for tests and
    tuning sweeps only: every plan computes the same operator."""
    st = load().gla_plan_override(PLAN_KNOBS[knob], int(value))
    if st != 0:
        raise GlaError(st, "gla_plan_override")


PLAN_FIELDS = ("seg_len", "segs_item", "cps1", "chunk1", "cps2", "chunk2", "pass1_reg", "pass2_heads", "rope_lds1",
               "rope_lds2")
_FORMS = {"bidirectional": 0, "block_causal": 1, "token_causal": 2}


def plan_describe(form: str, grid, heads: int, d: int, dtype: int, batch: int = 1, block_frames: int = 1) -> dict:
    """The launch plan a call with these shapes would use under the current
    knobs (PLAN_FIELDS; pass2_heads 0 means one head per workgroup).  For
    tests; needs no device."""
    T, H, W = (int(x) for x in grid)
    out = (ctypes.c_int * len(PLAN_FIELDS))()
    st = load().gla_plan_describe(_FORMS[form], int(batch), T, H, W, int(heads), int(d), int(dtype),
                                  int(block_frames), out, len(PLAN_FIELDS))
    if st != 0:
        raise GlaError(st, "gla_plan_describe")
    return dict(zip(PLAN_FIELDS, out))


def plan_reset() -> None:
    """Restore the default launch plan for every knob."""
    for knob in PLAN_KNOBS:
        plan_override(knob, 0)


def timing_enable(on: bool = True) -> None:
    st = load().gla_timing_enable(1 if on else 0)
    if st != 0:
        raise GlaError(st, "gla_timing_enable")


def timing_select(kernels=None) -> None:
    """Time only the named kernels (gla_kernel_name names, or ids); None: all."""
    lib = load()
    if kernels is None:
        mask = 0xFFFFFFFF
    else:
        names = [lib.gla_kernel_name(i).decode() for i in range(NUM_KERNELS)]
        mask = 0
        for k in kernels:
            mask |= 1 << (names.index(k) if isinstance(k, str) else int(k))
    st = lib.gla_timing_select(mask)
    if st != 0:
        raise GlaError(st, "gla_timing_select")


def timing_read() -> dict:
    """Per-kernel (milliseconds, launches) accumulated since the last read."""
    lib = load()
    ms = (ctypes.c_double * NUM_KERNELS)()
    n = (ctypes.c_longlong * NUM_KERNELS)()
    st = lib.gla_timing_read(ms, n, NUM_KERNELS)
    if st != 0:
        raise GlaError(st, "gla_timing_read")
    return {lib.gla_kernel_name(i).decode(): (ms[i], int(n[i])) for i in range(NUM_KERNELS)}
