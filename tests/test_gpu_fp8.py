"""GPU parity of the FP8 E4M3 operator I/O (q, k, v, g, beta and out in OCP
e4m3fn; fp32 state and accumulation) against the fp64 oracle evaluated on the
exact decoded fp8 inputs.  The output is compared beyond its own rounding:
|got - ref| - 2^-4 |ref| - 2^-10 <= 2e-2 max|ref| (the bf16 tolerance for the
path's internal error)."""
import dataclasses

import numpy as np
import pytest

import oracle.gla_oracle as orc
from workloads import WORKLOADS, fp8_bits_to_f32, head_slice_f32, make_inputs, make_state, make_workload_inputs
from tests.gpu_helpers import (TOL, Z_TOL, fp8_excess, grouped_head_error, rel_err, run_block_causal, run_forward,
                               to_device, to_f64)

pytestmark = pytest.mark.gpu


def _oracle(inp, **kw):
    return orc.gla_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"], inp["grid"],
                           inp["eps"], **kw)


def _oracle_bc(inp, F, S0=None, z0=None, **kw):
    return orc.gla_block_causal_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"],
                                        inp["grid"], inp["eps"], F, S0=S0, z0=z0, **kw)


def _report(name, err):
    print(f"[parity] fp8 {name}: error beyond output rounding {err:.3e} (tol {TOL['fp8']:.0e})", flush=True)


@pytest.mark.parametrize("shape", [(2, 4, 4, 2, 32), (1, 1, 1, 3, 64), (3, 5, 7, 2, 64), (5, 9, 13, 3, 128),
                                   (4, 16, 16, 2, 128), (9, 15, 26, 2, 64), (5, 9, 13, 4, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_shapes(shape):
    T, H, W, heads, d = shape
    print(f"[case] fp8 shape {shape}", flush=True)
    inp = make_inputs(T, H, W, heads, d, "fp8", seed=31)
    out = run_forward(to_device(inp), inp["grid"], inp["eps"])
    got = to_f64(out)
    ref = _oracle(inp)
    err = fp8_excess(got, ref)
    _report(str(shape), err)
    assert np.all(np.isfinite(got))
    assert err <= TOL["fp8"]


def test_fp8_480p_workload():
    w = WORKLOADS["480p"]
    print(f"[case] fp8 {w.name}", flush=True)
    inp = make_inputs(w.T, w.H, w.W, w.heads, w.d, "fp8", seed=0, eps=w.eps)
    got = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = fp8_excess(got, _oracle(inp))
    _report(w.name, err)
    assert err <= TOL["fp8"]


def test_fp8_long_sequence_full():
    """720p/60s with fp8 I/O at full size (N = 159,280, 32 heads; the launch
    plan the fp8 bench line times): every output of every head against the
    oracle on the decoded fp8 inputs, 8 heads per oracle call."""
    torch = pytest.importorskip("torch")
    w = dataclasses.replace(WORKLOADS["720p_60s"], dtype="fp8")
    print(f"[case] fp8 {w.name} N={w.N} heads={w.heads}", flush=True)
    inp = make_workload_inputs(w, seed=0, keep_f32=False)
    dev = to_device(inp)
    out = run_forward(dev, inp["grid"], inp["eps"])
    del dev
    assert bool(torch.isfinite(out.float()).all())
    err = grouped_head_error(out, inp, lambda sub: _oracle(sub), kind="fp8", label="fp8 " + w.name)
    _report(w.name + " all heads, all rows", err)
    assert err <= TOL["fp8"]


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_every_gate_code(d):
    """Gates running through every finite e4m3 code (both signs, subnormals up
    to +-448, the two NaN codes left out), so the gate's sigmoid is checked at
    every input the format has, saturated ends included."""
    T, H, W, heads = 4, 8, 9, 2
    inp = make_inputs(T, H, W, heads, d, "fp8", seed=41)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    n = inp["g_bits"].size
    bits = np.resize(np.random.default_rng(5).permutation(codes), n).reshape(inp["g_bits"].shape)
    inp["g_bits"] = bits
    inp["g"] = fp8_bits_to_f32(bits)
    assert set(np.unique(bits)) == set(codes)
    got = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = fp8_excess(got, _oracle(inp))
    _report(f"every gate code d={d}", err)
    assert np.all(np.isfinite(got))
    assert err <= TOL["fp8"]


@pytest.mark.parametrize("shape", [(7, 3, 5, 2, 64, 2), (9, 8, 9, 2, 128, 3)], ids=lambda s: "x".join(map(str, s)))
def test_fp8_block_causal(shape):
    T, H, W, heads, d, F = shape
    print(f"[case] fp8 block-causal {shape}", flush=True)
    inp = make_inputs(T, H, W, heads, d, "fp8", seed=32)
    S0, z0 = make_state(heads, d, seed=4)
    out, S, z = run_block_causal(to_device(inp), inp["grid"], inp["eps"], F, S0, z0)
    ro, rS, rz = _oracle_bc(inp, F, S0=S0, z0=z0)
    err = fp8_excess(to_f64(out), ro)
    _report(f"block-causal {shape}", err)
    assert err <= TOL["fp8"]
    assert rel_err(to_f64(S), rS) <= 1e-2
    assert rel_err(to_f64(z), rz) <= Z_TOL["fp8"]


def test_fp8_streamed_calls():
    T, H, W, heads, d, F = 6, 5, 6, 2, 128, 2
    hw = H * W
    inp = make_inputs(T, H, W, heads, d, "fp8", seed=33)
    outs, S, z = [], None, None
    for t0, t1 in ((0, 2), (2, 6)):
        part = {k: (v[t0 * hw: t1 * hw] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in inp.items()}
        part["grid"] = (t1 - t0, H, W)
        o, S_t, z_t = run_block_causal(to_device(part), part["grid"], part["eps"], F, S, z, t_offset=t0)
        outs.append(to_f64(o))
        S, z = S_t.cpu().numpy(), z_t.cpu().numpy()
    ro, rS, rz = _oracle_bc(inp, F)
    err = fp8_excess(np.concatenate(outs), ro)
    _report("streamed", err)
    assert err <= TOL["fp8"]
    assert rel_err(S.astype(np.float64), rS) <= 1e-2


def test_fp8_binding_rejects_mixed_dtypes():
    torch = pytest.importorskip("torch")
    import gated_bidirectional_linear_amd as gla
    inp = make_inputs(2, 2, 2, 2, 32, "fp8", seed=34)
    dev = to_device(inp)
    dev["g"] = dev["g"].to(torch.bfloat16)
    with pytest.raises(TypeError):
        gla.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], inp["grid"])


@pytest.mark.parametrize("d", [128])
def test_fp8_every_gate_code_four_heads(plan, d):
    """Every finite e4m3 gate code through the four-head output kernel (the
    fp8 default for head counts divisible by 4), whose stream waves look
    sigmoid(g) up in the LDS table of the 256 codes."""
    plan("pass2_heads", 4)
    T, H, W, heads = 4, 8, 9, 4
    inp = make_inputs(T, H, W, heads, d, "fp8", seed=42)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    n = inp["g_bits"].size
    bits = np.resize(np.random.default_rng(6).permutation(codes), n).reshape(inp["g_bits"].shape)
    inp["g_bits"] = bits
    inp["g"] = fp8_bits_to_f32(bits)
    got = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = fp8_excess(got, _oracle(inp))
    _report(f"every gate code, four heads, d={d}", err)
    assert np.all(np.isfinite(got))
    assert err <= TOL["fp8"]


@pytest.mark.parametrize("shape", [(5, 9, 13, 4, 128), (1, 1, 1, 8, 128), (2, 5, 9, 12, 128)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("heads_per_wg", [4, 1])
def test_fp8_four_head_kernel_shapes(plan, shape, heads_per_wg):
    """The four-head output kernel on fp8 rows (512-byte token segments; its
    MFMA waves compute the features), and the one-head kernel on the same
    shapes (chosen by the plan knob)."""
    plan("pass2_heads", heads_per_wg)
    T, H, W, heads, d = shape
    inp = make_inputs(T, H, W, heads, d, "fp8", seed=44)
    got = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = fp8_excess(got, _oracle(inp))
    _report(f"{heads_per_wg}-head kernel {shape}", err)
    assert np.all(np.isfinite(got))
    assert err <= TOL["fp8"]


def test_fp8_block_causal_four_heads(plan):
    """Block-causal fp8 with 8 heads: per-block states through the four-head kernel."""
    plan("pass2_heads", 4)
    T, H, W, heads, d, F = 7, 6, 7, 8, 128, 3
    inp = make_inputs(T, H, W, heads, d, "fp8", seed=43)
    S0, z0 = make_state(heads, d, seed=8)
    out, S, z = run_block_causal(to_device(inp), inp["grid"], inp["eps"], F, S0, z0)
    ro, rS, rz = _oracle_bc(inp, F, S0=S0, z0=z0)
    err = fp8_excess(to_f64(out), ro)
    _report(f"block-causal four heads {(T, H, W, heads, F)}", err)
    assert err <= TOL["fp8"]
    assert rel_err(to_f64(z), rz) <= Z_TOL["fp8"]


@pytest.mark.parametrize("fmt", ["fp8", "e5m2"])
def test_fp8_wide_frame_rope_rows_in_lds(fmt):
    """34 x 60 latent frames (1080p): y and x RoPE blocks of 2,256 entries
    staged in LDS for the register pass 1 and the four-head output kernel."""
    import gated_bidirectional_linear_amd as gla
    code = gla.DTYPE_FP8_E4M3 if fmt == "fp8" else gla.DTYPE_FP8_E5M2
    p = gla.plan_describe("bidirectional", (3, 34, 60), 4, 128, code)
    assert (p["rope_lds1"], p["rope_lds2"], p["pass1_reg"], p["pass2_heads"]) == (1, 1, 1, 4)
    inp = make_inputs(3, 34, 60, 4, 128, fmt, seed=45)
    got = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = fp8_excess(got, _oracle(inp), fmt)
    _report(f"wide frame {fmt}", err)
    assert np.all(np.isfinite(got))
    assert err <= TOL[fmt]
