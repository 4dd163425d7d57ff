"""GPU parity of the FP8 E5M2 operator I/O (q, k, v, g, beta and out in OCP
E5M2; fp32 state and accumulation) against the fp64 oracle evaluated on the
exact decoded e5m2 inputs.  The output is compared beyond its own rounding:
|got - ref| - 2^-3 |ref| - 2^-17 <= 2e-2 max|ref| (the bf16 tolerance for the
path's internal error)."""
import numpy as np
import pytest

import oracle.gla_oracle as orc
from workloads import WORKLOADS, e5m2_bits_to_f32, make_inputs, make_state
from tests.gpu_helpers import (TOL, Z_TOL, fp8_excess, rel_err, run_block_causal, run_forward, to_device, to_f64)

pytestmark = pytest.mark.gpu


def _oracle(inp, **kw):
    return orc.gla_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"], inp["grid"],
                           inp["eps"], **kw)


def _oracle_bc(inp, F, S0=None, z0=None, **kw):
    return orc.gla_block_causal_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"],
                                        inp["grid"], inp["eps"], F, S0=S0, z0=z0, **kw)


def _check_out(name, got, ref):
    err = fp8_excess(got, ref, "e5m2")
    print(f"[parity] e5m2 {name}: error beyond output rounding {err:.3e} (tol {TOL['e5m2']:.0e})", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= TOL["e5m2"]


@pytest.mark.parametrize("shape", [(2, 4, 4, 2, 32), (1, 1, 1, 3, 64), (3, 5, 7, 2, 64), (5, 9, 13, 3, 128),
                                   (4, 16, 16, 2, 128), (5, 9, 13, 4, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_e5m2_shapes(shape):
    T, H, W, heads, d = shape
    print(f"[case] e5m2 shape {shape}", flush=True)
    inp = make_inputs(T, H, W, heads, d, "e5m2", seed=61)
    _check_out(str(shape), to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"])), _oracle(inp))


def test_e5m2_480p_workload():
    w = WORKLOADS["480p"]
    print(f"[case] e5m2 {w.name}", flush=True)
    inp = make_inputs(w.T, w.H, w.W, w.heads, w.d, "e5m2", seed=0, eps=w.eps)
    _check_out(w.name, to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"])), _oracle(inp))


def _every_gate_code(seed, heads, d):
    T, H, W = 4, 8, 9
    inp = make_inputs(T, H, W, heads, d, "e5m2", seed=seed)
    codes = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], dtype=np.uint8)   # every finite code
    n = inp["g_bits"].size
    bits = np.resize(np.random.default_rng(seed).permutation(codes), n).reshape(inp["g_bits"].shape)
    inp["g_bits"] = bits
    inp["g"] = e5m2_bits_to_f32(bits)
    assert set(np.unique(bits)) == set(codes)
    return inp


@pytest.mark.parametrize("d", [64, 128])
def test_e5m2_every_gate_code(d):
    """Gates running through every finite e5m2 code (both signs, subnormals up
    to +-57344), so the gate's sigmoid is checked at every finite input the
    format has, saturated ends included."""
    inp = _every_gate_code(62, 2, d)
    _check_out(f"every gate code d={d}", to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"])), _oracle(inp))


def test_e5m2_every_gate_code_four_heads(plan):
    """The same through the four-head output kernel (chosen by the plan knob)."""
    plan("pass2_heads", 4)
    inp = _every_gate_code(63, 4, 128)
    _check_out("every gate code, four heads", to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"])),
               _oracle(inp))


@pytest.mark.parametrize("shape", [(5, 9, 13, 4, 128), (2, 5, 9, 12, 128)], ids=lambda s: "x".join(map(str, s)))
def test_e5m2_four_head_kernel_shapes(plan, shape):
    plan("pass2_heads", 4)
    T, H, W, heads, d = shape
    inp = make_inputs(T, H, W, heads, d, "e5m2", seed=64)
    _check_out(f"four-head kernel {shape}", to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"])),
               _oracle(inp))


def test_e5m2_wide_input_scale():
    """Inputs spread over 2^-12 .. 2^12 (outside what e4m3 holds at either
    end): q, k, v scaled per token by powers of two, so the key and value
    rows span the format's range; the output is scale-free (RMSNorm)."""
    T, H, W, heads, d = 3, 6, 7, 2, 128
    inp = make_inputs(T, H, W, heads, d, "f32", seed=65)
    rng = np.random.default_rng(65)
    from workloads import f32_to_e5m2_bits
    N = T * H * W
    for name in ("q", "k", "v"):
        scale = np.exp2(rng.integers(-12, 13, size=(N, heads, 1))).astype(np.float64)
        bits = f32_to_e5m2_bits(inp[name] * scale)
        inp[name + "_bits"] = bits
        inp[name] = e5m2_bits_to_f32(bits)
    for name in ("g", "beta"):
        bits = f32_to_e5m2_bits(inp[name])
        inp[name + "_bits"] = bits
        inp[name] = e5m2_bits_to_f32(bits)
    inp["dtype"] = "e5m2"
    _check_out("wide input scale", to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"])), _oracle(inp))


@pytest.mark.parametrize("shape", [(7, 3, 5, 2, 64, 2), (9, 8, 9, 2, 128, 3)], ids=lambda s: "x".join(map(str, s)))
def test_e5m2_block_causal(shape):
    T, H, W, heads, d, F = shape
    print(f"[case] e5m2 block-causal {shape}", flush=True)
    inp = make_inputs(T, H, W, heads, d, "e5m2", seed=66)
    S0, z0 = make_state(heads, d, seed=6)
    out, S, z = run_block_causal(to_device(inp), inp["grid"], inp["eps"], F, S0, z0)
    ro, rS, rz = _oracle_bc(inp, F, S0=S0, z0=z0)
    _check_out(f"block-causal {shape}", to_f64(out), ro)
    assert rel_err(to_f64(S), rS) <= 1e-2
    assert rel_err(to_f64(z), rz) <= Z_TOL["e5m2"]


def test_e5m2_binding_rejects_mixed_fp8_formats():
    torch = pytest.importorskip("torch")
    import gated_bidirectional_linear_amd as gla
    inp = make_inputs(2, 2, 2, 2, 32, "e5m2", seed=67)
    dev = to_device(inp)
    dev["k"] = dev["k"].view(torch.uint8).view(torch.float8_e4m3fn)
    with pytest.raises(TypeError):
        gla.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], inp["grid"])
