"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 2e-2, "e5m2": 2e-2}   # max|err| <= TOL * max|ref| (fp8, e5m2: beyond
# the output's own rounding)

# Rounding of an fp8 output to nearest: at most REL * |x| for normal values and
# ABS below the smallest normal (half a unit of the last place).
FP8_ROUNDING = {"fp8": (2.0 ** -4, 2.0 ** -10), "e5m2": (2.0 ** -3, 2.0 ** -17)}

# Key-sum state z.  For bf16 inputs the HIP path multiplies each token's phi(k)
# by its RMS factor rounded to bf16 (relative error <= 2^-9); every term of z
# is non-negative, so each channel's sum keeps that relative bound.  fp32
# accumulation over the sequence adds far less.
Z_TOL = {"f32": 1e-5, "bf16": 2.5e-3, "fp8": 2.5e-3, "e5m2": 2.5e-3}   # fp8 at d = 128 runs the bf16 fast pass 1 too


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
        elif inp["dtype"] in ("fp8", "e5m2"):
            bits = np.ascontiguousarray(inp[name + "_bits"], dtype=np.uint8)
            tdt = torch.float8_e4m3fn if inp["dtype"] == "fp8" else torch.float8_e5m2
            out[name] = torch.from_numpy(bits).to(device).view(tdt)
        else:
            out[name] = torch.from_numpy(np.ascontiguousarray(inp[name])).to(device)
    out["rms_w"] = torch.from_numpy(np.ascontiguousarray(inp["rms_w"], dtype=np.float32)).to(device)
    return out


def to_f64(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):   # decoded by the generator's own codecs
        from workloads import e5m2_bits_to_f32, fp8_bits_to_f32
        decode = fp8_bits_to_f32 if t.dtype == torch.float8_e4m3fn else e5m2_bits_to_f32
        return decode(t.detach().view(torch.uint8).cpu().numpy()).astype(np.float64)
    return t.detach().to(torch.float64).cpu().numpy()


def fp8_excess(got, ref, fmt="fp8") -> float:
    """Error of an FP8 output beyond its own rounding, relative to max|ref|:
    max(|got - ref| - REL |ref| - ABS) / max|ref| with (REL, ABS) from
    FP8_ROUNDING (E4M3: 2^-4 for normal values, 2^-10 below 2^-6; E5M2: 2^-3,
    2^-17 below 2^-14); what is left is the path's internal error, held to the
    bf16 tolerance."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    rel, ab = FP8_ROUNDING[fmt]
    ex = np.abs(got - ref) - rel * np.abs(ref) - ab
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


def grouped_head_error(out, inp, ref_fn, kind="rel", rows=None, group=8, label=""):
    """Error of a full-size GPU output over every head, against the oracle run
    on `group` heads at a time (bounded host memory).

    out    : GPU output [N, heads, d]
    inp    : a bits-only bf16 or fp8 input set (make_inputs(..., keep_f32=False))
    ref_fn : oracle call on an input set holding only the group's heads;
             returns [len(rows) or N, group, d]
    kind   : "rel" -> max|got - ref| / max|ref|; "fp8" or "e5m2" ->
             fp8_excess's numerator over max|ref|, both maxima over all heads
    rows   : token rows compared (None: every row)
    """
    from workloads import head_slice_f32
    torch = torch_mod()
    heads = out.shape[1]
    worst, top = 0.0, 0.0
    idx = None if rows is None else torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(out.device)
    for h0 in range(0, heads, group):
        hs = list(range(h0, min(h0 + group, heads)))
        ref = np.asarray(ref_fn(head_slice_f32(inp, hs)), np.float64)
        sel = out[:, h0:h0 + len(hs), :] if idx is None else out[idx][:, h0:h0 + len(hs), :]
        got = to_f64(sel)
        if kind in FP8_ROUNDING:
            rel, ab = FP8_ROUNDING[kind]
            ex = np.abs(got - ref) - rel * np.abs(ref) - ab
            worst = max(worst, float(np.max(ex)))
        else:
            worst = max(worst, float(np.max(np.abs(got - ref))))
        top = max(top, float(np.max(np.abs(ref))))
        print(f"[parity] {label} heads {hs[0]}..{hs[-1]}: running error {max(worst, 0.0) / max(top, 1e-300):.3e}",
              flush=True)
        del ref, got
    return max(worst, 0.0) / (top if top > 0 else 1.0)
