"""Seeded synthetic inputs for the gated bidirectional linear-attention operator.

This module is shared by the tests, the benchmark and the smoke check. It holds
only input construction: the workload table (grid, heads, head dim, dtype,
block size), seeded random draws, and the storage conversion of fp32 draws to
bfloat16 and fp8 bits. None of the operator's arithmetic lives here.

Workload shapes follow the pages' video-latent grids (SANA-Video 2.0 digest,
"results" table and the 480p/720p workloads; SANA-Video notes, block linear
attention): 480p/81 frames is an 11x15x26 latent grid (4,290 tokens), 720p is
22x40 latent pixels per frame, and 60 s at 24 fps gives 181 latent frames.

Draw recipe: q, k, v, g ~ N(0,1) fp32, beta = sigmoid(N(0,1)), rms_w =
1 + 0.1*N(0,1) fp32, every tensor from its own counter-keyed PCG64 streams
(see make_inputs).  For bf16 workloads every tensor handed to the operator
(q, k, v, g, beta) is rounded to bfloat16 with round-to-nearest-even; rms_w
stays fp32.  fp8 (OCP E4M3) and e5m2 (OCP E5M2) workloads round the same
tensors to their format the same way.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "round_to_bf16",
    "f32_to_fp8_bits",
    "fp8_bits_to_f32",
    "round_to_fp8",
    "FP8_MAX",
    "f32_to_e5m2_bits",
    "e5m2_bits_to_f32",
    "round_to_e5m2",
    "E5M2_MAX",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    W: int
    heads: int
    d: int
    dtype: str  # "f32", "bf16", "fp8" (OCP E4M3) or "e5m2" (OCP E5M2)
    block_frames: Optional[int] = None  # None: bidirectional
    eps: float = 1e-6

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def elem_size(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1, "e5m2": 1}[self.dtype]

    def alg_bytes(self) -> int:
        """Algorithmic HBM bytes of one call: read q,k,v,g,beta, write out,
        plus read+write of the fp32 carried state in block-causal mode."""
        s = self.elem_size
        b = 5 * self.N * self.heads * self.d * s + self.N * self.heads * s
        if self.block_frames is not None:
            b += 2 * self.heads * (self.d * self.d + self.d) * 4
        return b

    def alg_flops(self) -> int:
        return 4 * self.N * self.heads * self.d * self.d


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32", 2, 4, 4, 2, 32, "f32"),
        Workload("480p", 11, 15, 26, 20, 128, "bf16"),
        Workload("720p_5s_h20", 16, 22, 40, 20, 128, "bf16"),
        Workload("720p_5s_h32", 16, 22, 40, 32, 128, "bf16"),
        Workload("720p_60s", 181, 22, 40, 32, 128, "bf16"),
        Workload("block_causal_720p", 24, 22, 40, 20, 128, "bf16", block_frames=3),
        Workload("1080p_121f", 16, 34, 60, 32, 128, "bf16"),
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round-to-nearest-even); returns uint16 bits.

    Inputs here are finite draws, so NaN handling is not needed; infinities and
    overflow to infinity follow the same integer rounding rule.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value, returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits;
# exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; there are no
# infinities and the largest finite value is 448 (S.1111.110).
FP8_MAX = 448.0


def fp8_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode FP8 E4M3 bits (uint8) to fp32 values."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int32)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((b & 7) == 7), np.nan, mag)
    return np.where(b & 0x80, -mag, mag).astype(np.float32)


def f32_to_fp8_bits(x: np.ndarray) -> np.ndarray:
    """Round values to FP8 E4M3, nearest with ties to even, saturating
    magnitudes past 448 to 448; returns uint8 bits.  Inputs must not be NaN."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int32)
    # subnormal range (a < 2^-6): units of 2^-9; 8 units is the smallest normal (code 8)
    sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    # normal range: a = f * 2^ex with f in [0.5, 1), exponent e = ex - 1
    f, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = ex.astype(np.int64) - 1
    q = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)   # 0..8 eighths above 1
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    norm = ((e + 7) << 3) | q
    code = np.where(a < 2.0 ** -6, sub, norm)
    code = np.where(a >= FP8_MAX, 0x7E, np.minimum(code, 0x7E))
    return (code.astype(np.int32) | sign).astype(np.uint8)


def round_to_fp8(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest FP8 E4M3 value, returned as fp32."""
    return fp8_bits_to_f32(f32_to_fp8_bits(x))


# OCP FP8 E5M2: sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent
# field 0 holds subnormals m * 2^-16; exponent field 31 holds +-infinity
# (mantissa 0) and NaN; the largest finite value is 57344 (S.11110.11).
E5M2_MAX = 57344.0


def e5m2_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode FP8 E5M2 bits (uint8) to fp32 values."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int32)
    e = (b >> 2) & 0x1F
    m = b & 3
    mag = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.exp2(e.astype(np.float64) - 15.0))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(b & 0x80, -mag, mag).astype(np.float32)


def f32_to_e5m2_bits(x: np.ndarray) -> np.ndarray:
    """Round finite values to FP8 E5M2, nearest with ties to even, saturating
    magnitudes past 57344 to 57344; returns uint8 bits.  Inputs must be finite."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int32)
    # subnormal range (a < 2^-14): units of 2^-16; 4 units is the smallest normal (code 4)
    sub = np.rint(a * 2.0 ** 16).astype(np.int64)
    f, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = ex.astype(np.int64) - 1
    q = np.rint((2.0 * f - 1.0) * 4.0).astype(np.int64)   # 0..4 quarters above 1
    e = np.where(q == 4, e + 1, e)
    q = np.where(q == 4, 0, q)
    norm = (np.clip(e + 15, 0, 31) << 2) | q
    code = np.where(a < 2.0 ** -14, sub, norm)
    code = np.where(a >= E5M2_MAX, 0x7B, np.minimum(code, 0x7B))
    return (code.astype(np.int32) | sign).astype(np.uint8)


def round_to_e5m2(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest FP8 E5M2 value, returned as fp32."""
    return e5m2_bits_to_f32(f32_to_e5m2_bits(x))


# storage codecs of the narrow dtypes: (numpy storage type, encode, decode)
CODECS = {
    "bf16": (np.uint16, f32_to_bf16_bits, bf16_bits_to_f32),
    "fp8": (np.uint8, f32_to_fp8_bits, fp8_bits_to_f32),
    "e5m2": (np.uint8, f32_to_e5m2_bits, e5m2_bits_to_f32),
}


_BLOCK = 1 << 22          # elements per independently seeded block
_STREAMS = {"q": 0, "k": 1, "v": 2, "g": 3, "beta": 4, "rms_w": 5}


def _normal_block(seed: int, stream: int, block: int, n: int) -> np.ndarray:
    ss = np.random.SeedSequence(seed, spawn_key=(stream, block))
    return np.random.Generator(np.random.PCG64(ss)).standard_normal(n, dtype=np.float32)


def _workers() -> int:
    try:
        import os
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = 4
    return max(1, min(16, n))


def _codec(dtype: str):
    """(encode, decode) of a narrow storage dtype."""
    return CODECS[dtype][1], CODECS[dtype][2]


def _draw(seed: int, name: str, shape, dtype: str, keep_f32: bool, pool, sigmoid: bool = False):
    size = int(np.prod(shape))
    f32 = np.empty(size, np.float32) if (keep_f32 or dtype == "f32") else None
    bits = np.empty(size, CODECS[dtype][0]) if dtype != "f32" else None
    encode, decode = _codec(dtype) if dtype != "f32" else (None, None)
    stream = _STREAMS[name]

    def work(b):
        lo = b * _BLOCK
        hi = min(size, lo + _BLOCK)
        x = _normal_block(seed, stream, b, hi - lo)
        if sigmoid:
            x = (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)
        if bits is not None:
            bb = encode(x)
            bits[lo:hi] = bb
            if f32 is not None:
                f32[lo:hi] = decode(bb)
        else:
            f32[lo:hi] = x

    nblocks = (size + _BLOCK - 1) // _BLOCK
    if pool is None or nblocks <= 1:
        for b in range(nblocks):
            work(b)
    else:
        list(pool.map(work, range(nblocks)))
    return (None if f32 is None else f32.reshape(shape)), (None if bits is None else bits.reshape(shape))


def make_inputs(T: int, H: int, W: int, heads: int, d: int, dtype: str, seed: int = 0,
                eps: float = 1e-6, keep_f32: bool = True) -> dict:
    """Draw one seeded input set.

    Returns a dict with fp32 numpy arrays ``q, k, v, g`` of shape [N, heads, d],
    ``beta`` [N, heads], ``rms_w`` [d], plus ``eps``, ``grid`` (T, H, W) and
    ``dtype``.  For dtype "bf16" ("fp8", "e5m2") the fp32 arrays hold exactly
    the bf16 (FP8 E4M3, FP8 E5M2) values the operator receives, and ``*_bits``
    (uint16, uint8) hold their storage; with keep_f32=False only the bits are
    kept (large workloads).

    Each tensor is filled in row-major order in blocks of 2^22 elements; block
    b of tensor t (q, k, v, g, beta-logit, rms_w-noise = 0..5) is drawn from
    PCG64(SeedSequence(seed, spawn_key=(t, b))), so the values do not depend
    on how many threads draw them.
    """
    if dtype not in ("f32", "bf16", "fp8", "e5m2"):
        raise ValueError(f"unknown dtype {dtype!r}")
    N = T * H * W
    from concurrent.futures import ThreadPoolExecutor
    out = {}
    big = N * heads * d > 2 * _BLOCK
    pool = ThreadPoolExecutor(_workers()) if big else None
    try:
        for name in ("q", "k", "v", "g"):
            f, b = _draw(seed, name, (N, heads, d), dtype, keep_f32, pool)
            out[name] = f
            if b is not None:
                out[name + "_bits"] = b
        f, b = _draw(seed, "beta", (N, heads), dtype, keep_f32, pool, sigmoid=True)
        out["beta"] = f
        if b is not None:
            out["beta_bits"] = b
    finally:
        if pool is not None:
            pool.shutdown()
    noise = _normal_block(seed, _STREAMS["rms_w"], 0, d)
    out["rms_w"] = (1.0 + 0.1 * noise.astype(np.float64)).astype(np.float32)
    out["eps"] = float(eps)
    out["grid"] = (T, H, W)
    out["dtype"] = dtype
    return out


def make_workload_inputs(w: Workload, seed: int = 0, keep_f32: bool = True) -> dict:
    return make_inputs(w.T, w.H, w.W, w.heads, w.d, w.dtype, seed=seed, eps=w.eps, keep_f32=keep_f32)


def head_slice_f32(inp: dict, heads) -> dict:
    """fp32 copies of the listed heads of a bits-only bf16 or fp8 input set."""
    out = dict(inp)
    decode = _codec(inp["dtype"])[1]
    for name in ("q", "k", "v", "g"):
        out[name] = decode(inp[name + "_bits"][:, heads, :])
    out["beta"] = decode(inp["beta_bits"][:, heads])
    return out


def make_state(heads: int, d: int, seed: int, scale: float = 1.0) -> tuple:
    """A seeded carried state (S [heads,d,d], z [heads,d]) for block-causal tests.

    z is drawn non-negative, as a key sum of ReLU features always is.
    """
    rng = np.random.default_rng(seed)
    S = (scale * rng.standard_normal((heads, d, d))).astype(np.float32)
    z = (scale * np.abs(rng.standard_normal((heads, d)))).astype(np.float32)
    return S, z
