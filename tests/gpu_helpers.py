"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 2e-2}   # max|err| <= TOL * max|ref| (fp8: beyond output rounding)

# Key-sum state z.  For bf16 inputs the HIP path multiplies each token's phi(k)
# by its RMS factor rounded to bf16 (relative error <= 2^-9); every term of z
# is non-negative, so each channel's sum keeps that relative bound.  fp32
# accumulation over the sequence adds far less.
Z_TOL = {"f32": 1e-5, "bf16": 2.5e-3, "fp8": 2.5e-3}   # fp8 at d = 128 runs the bf16 fast pass 1 too


def torch_mod():
    import torch
    return torch


def gpu_available() -> bool:
    try:
        torch = torch_mod()
        return torch.cuda.is_available()
    except Exception:
        return False


def to_device(inp: dict, device="cuda"):
    """Upload a make_inputs() dict: bf16 and fp8 from their exact bits, f32 as is."""
    torch = torch_mod()
    out = {}
    for name in ("q", "k", "v", "g", "beta"):
        if inp["dtype"] == "bf16":
            bits = np.ascontiguousarray(inp[name + "_bits"]).view(np.int16)
            out[name] = torch.from_numpy(bits).to(device).view(torch.bfloat16)
        elif inp["dtype"] == "fp8":
            bits = np.ascontiguousarray(inp[name + "_bits"], dtype=np.uint8)
            out[name] = torch.from_numpy(bits).to(device).view(torch.float8_e4m3fn)
        else:
            out[name] = torch.from_numpy(np.ascontiguousarray(inp[name])).to(device)
    out["rms_w"] = torch.from_numpy(np.ascontiguousarray(inp["rms_w"], dtype=np.float32)).to(device)
    return out


def to_f64(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.float8_e4m3fn:   # decoded by the generator's own codec
        from workloads import fp8_bits_to_f32
        return fp8_bits_to_f32(t.detach().view(torch.uint8).cpu().numpy()).astype(np.float64)
    return t.detach().to(torch.float64).cpu().numpy()


def fp8_excess(got, ref) -> float:
    """Error of an FP8 E4M3 output beyond its own rounding, relative to max|ref|:
    max(|got - ref| - 2^-4 |ref| - 2^-10) / max|ref|.  Rounding to nearest
    costs at most 2^-4 |x| for normal values and 2^-10 below 2^-6; what is
    left is the path's internal error, held to the bf16 tolerance."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    ex = np.abs(got - ref) - 2.0 ** -4 * np.abs(ref) - 2.0 ** -10
    return max(0.0, float(np.max(ex))) / (den if den > 0 else 1.0)


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (den if den > 0 else 1.0)


def run_forward(dev: dict, grid, eps):
    import gated_bidirectional_linear_amd as gla
    torch = torch_mod()
    out = gla.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], grid, eps=eps)
    torch.cuda.synchronize()
    return out


def run_block_causal(dev: dict, grid, eps, block_frames, S0=None, z0=None, t_offset=0):
    import gated_bidirectional_linear_amd as gla
    torch = torch_mod()
    N, heads, d = dev["q"].shape
    S = torch.zeros((heads, d, d), dtype=torch.float32, device=dev["q"].device)
    z = torch.zeros((heads, d), dtype=torch.float32, device=dev["q"].device)
    if S0 is not None:
        S.copy_(torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)))
        z.copy_(torch.from_numpy(np.ascontiguousarray(z0, dtype=np.float32)))
    out = gla.block_causal_forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], grid,
                                   S, z, block_frames, eps=eps, t_offset=t_offset)
    torch.cuda.synchronize()
    return out, S, z


def run_token_causal(dev: dict, grid, eps, include_self=True, S0=None, z0=None, t_offset=0):
    import gated_bidirectional_linear_amd as gla
    torch = torch_mod()
    N, heads, d = dev["q"].shape
    S = torch.zeros((heads, d, d), dtype=torch.float32, device=dev["q"].device)
    z = torch.zeros((heads, d), dtype=torch.float32, device=dev["q"].device)
    if S0 is not None:
        S.copy_(torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)))
        z.copy_(torch.from_numpy(np.ascontiguousarray(z0, dtype=np.float32)))
    out = gla.token_causal_forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], grid,
                                   S, z, include_self=include_self, eps=eps, t_offset=t_offset)
    torch.cuda.synchronize()
    return out, S, z
