"""Seeded synthetic inputs for the gated bidirectional linear-attention operator.

This module is shared by the tests, the benchmark and the smoke check. It holds
only input construction: the workload table (grid, heads, head dim, dtype,
block size), seeded random draws, and the storage conversion of fp32 draws to
bfloat16 bits. None of the operator's arithmetic lives here.

Workload shapes follow the pages' video-latent grids (SANA-Video 2.0 digest,
"results" table and the 480p/720p workloads; SANA-Video notes, block linear
attention): 480p/81 frames is an 11x15x26 latent grid (4,290 tokens), 720p is
22x40 latent pixels per frame, and 60 s at 24 fps gives 181 latent frames.

Draw recipe (fixed order, one ``numpy.random.default_rng(seed)`` stream):
q, k, v, g ~ N(0,1) fp32, then beta-logits ~ N(0,1) fp32, then rms_w noise
~ N(0,1) fp32.  beta = sigmoid(logit), rms_w = 1 + 0.1*noise.  For bf16
workloads every tensor handed to the operator (q, k, v, g, beta) is rounded
to bfloat16 with round-to-nearest-even; rms_w stays fp32.
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
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    W: int
    heads: int
    d: int
    dtype: str  # "f32" or "bf16"
    block_frames: Optional[int] = None  # None: bidirectional
    eps: float = 1e-6

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    def alg_bytes(self) -> int:
        """Algorithmic HBM bytes of one call: read q,k,v,g,beta, write out,
        plus read+write of the fp32 carried state in block-causal mode."""
        s = 4 if self.dtype == "f32" else 2
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
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round-to-nearest-even); returns uint16 bits.

    Inputs here are finite draws, so NaN handling is not needed; infinities and
    overflow to infinity follow the same integer rounding rule.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value, returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def make_inputs(T: int, H: int, W: int, heads: int, d: int, dtype: str, seed: int = 0,
                eps: float = 1e-6) -> dict:
    """Draw one seeded input set.

    Returns a dict with fp32 numpy arrays ``q, k, v, g`` of shape [N, heads, d],
    ``beta`` [N, heads], ``rms_w`` [d], plus ``eps``, ``grid`` (T, H, W) and
    ``dtype``.  For dtype "bf16" the fp32 arrays hold exactly the bf16 values
    the operator receives, and ``*_bits`` (uint16) hold their storage.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    N = T * H * W
    rng = np.random.default_rng(seed)
    shape = (N, heads, d)
    out = {}
    for name in ("q", "k", "v", "g"):
        out[name] = rng.standard_normal(shape, dtype=np.float32)
    logits = rng.standard_normal((N, heads), dtype=np.float32)
    out["beta"] = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)
    noise = rng.standard_normal(d, dtype=np.float32)
    out["rms_w"] = (1.0 + 0.1 * noise.astype(np.float64)).astype(np.float32)
    if dtype == "bf16":
        for name in ("q", "k", "v", "g", "beta"):
            bits = f32_to_bf16_bits(out[name])
            out[name + "_bits"] = bits
            out[name] = bf16_bits_to_f32(bits)
    out["eps"] = float(eps)
    out["grid"] = (T, H, W)
    out["dtype"] = dtype
    return out


def make_workload_inputs(w: Workload, seed: int = 0) -> dict:
    return make_inputs(w.T, w.H, w.W, w.heads, w.d, w.dtype, seed=seed, eps=w.eps)


def make_state(heads: int, d: int, seed: int, scale: float = 1.0) -> tuple:
    """A seeded carried state (S [heads,d,d], z [heads,d]) for block-causal tests.

    z is drawn non-negative, as a key sum of ReLU features always is.
    """
    rng = np.random.default_rng(seed)
    S = (scale * rng.standard_normal((heads, d, d))).astype(np.float32)
    z = (scale * np.abs(rng.standard_normal((heads, d)))).astype(np.float32)
    return S, z
