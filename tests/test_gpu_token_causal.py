"""GPU parity of the token-level causal form: the HIP path (through the C ABI)
against the fp64 oracle, element by element on seeded inputs, for both
readings of whether a token reads its own contribution.

Tolerances as for the other forms: max|err| <= 1e-5 * max|ref| for fp32,
<= 2e-2 * max|ref| for bf16 (fp8: beyond the output's own rounding).
"""
import dataclasses

import numpy as np
import pytest

import oracle.gla_oracle as orc
from workloads import WORKLOADS, make_inputs, make_workload_inputs, make_state, head_slice_f32
from tests.gpu_helpers import (TOL, Z_TOL, to_device, to_f64, rel_err, fp8_excess, run_token_causal,
                               grouped_head_error)

pytestmark = pytest.mark.gpu

S_TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2, "e5m2": 1e-2}


def _oracle_tc(inp, include_self, S0=None, z0=None, **kw):
    return orc.gla_token_causal_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"],
                                        inp["grid"], inp["eps"], include_self=include_self, S0=S0, z0=z0, **kw)


def _out_err(got, ref, dtype):
    return fp8_excess(got, ref, dtype) if dtype in ("fp8", "e5m2") else rel_err(got, ref)


def _check(name, inp, include_self, S0=None, z0=None, t_offset=0):
    dtype = inp["dtype"]
    out, S, z = run_token_causal(to_device(inp), inp["grid"], inp["eps"], include_self, S0, z0, t_offset)
    ro, rS, rz = _oracle_tc(inp, include_self, S0, z0, pos_offset=(t_offset, 0, 0))
    o = to_f64(out)
    err = _out_err(o, ro, dtype)
    print(f"[parity] {name}: rel err {err:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert np.all(np.isfinite(o))
    assert err <= TOL[dtype]
    assert rel_err(to_f64(S), rS) <= S_TOL[dtype]
    assert rel_err(to_f64(z), rz) <= Z_TOL[dtype]
    return o


# (T, H, W, heads, d, dtype); N spans several 32-token tiles with a ragged tail
SHAPES = [
    (2, 4, 4, 2, 32, "f32"),     # the tiny configuration
    (3, 5, 7, 3, 64, "f32"),
    (2, 3, 5, 2, 128, "f32"),
    (3, 5, 7, 3, 64, "bf16"),
    (4, 6, 10, 4, 128, "bf16"),
    (3, 5, 7, 2, 32, "bf16"),
    (3, 4, 6, 3, 128, "bf16"),   # odd head count: one head per workgroup
    (3, 4, 5, 2, 128, "fp8"),
    (2, 5, 9, 2, 64, "fp8"),
    (3, 4, 5, 2, 128, "e5m2"),
    (2, 5, 9, 3, 64, "e5m2"),
]


@pytest.mark.parametrize("include_self", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_token_causal_shapes(shape, include_self):
    T, H, W, heads, d, dtype = shape
    print(f"[case] token-causal {shape} include_self={include_self}", flush=True)
    inp = make_inputs(T, H, W, heads, d, dtype, seed=31)
    _check(f"tc {shape} incl={include_self}", inp, include_self)


@pytest.mark.parametrize("wg", ["1", "3", "64"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_causal_segment_counts(plan, wg, dtype):
    """One segment walked by one workgroup per head, a few segments of many
    tiles, or many one-tile segments: the same result."""
    T, H, W, heads, d = 5, 7, 9, 2, 128
    plan("token_causal_workgroups", int(wg) * heads)
    print(f"[case] token-causal segments={wg} {dtype}", flush=True)
    inp = make_inputs(T, H, W, heads, d, dtype, seed=32)
    _check(f"tc segments {wg} {dtype}", inp, True)


@pytest.mark.parametrize("include_self", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_causal_carried_state(dtype, include_self):
    T, H, W, heads, d = 3, 6, 8, 2, 128
    print(f"[case] token-causal carried state {dtype} include_self={include_self}", flush=True)
    inp = make_inputs(T, H, W, heads, d, dtype, seed=33)
    S0, z0 = make_state(heads, d, seed=4, scale=3.0)
    _check(f"tc carried state {dtype} incl={include_self}", inp, include_self, S0, z0)


@pytest.mark.parametrize("include_self", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_causal_chained_calls(dtype, include_self):
    """A sequence streamed through calls on frame ranges, with frame offsets,
    gives the output and final state of one call (and of the oracle)."""
    T, H, W, heads, d = 7, 5, 6, 2, 64
    hw = H * W
    inp = make_inputs(T, H, W, heads, d, dtype, seed=34)
    one = _check(f"tc one call {dtype}", inp, include_self)
    S, z = None, None
    outs = []
    for t0, t1 in ((0, 2), (2, 3), (3, 7)):
        part = {k: (v[t0 * hw: t1 * hw] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in inp.items()}
        part["grid"] = (t1 - t0, H, W)
        o, S_t, z_t = run_token_causal(to_device(part), part["grid"], part["eps"], include_self, S, z, t_offset=t0)
        outs.append(to_f64(o))
        S, z = S_t.cpu().numpy(), z_t.cpu().numpy()
    chained = np.concatenate(outs)
    ro, rS, rz = _oracle_tc(inp, include_self)
    err = rel_err(chained, ro)
    print(f"[parity] tc chained {dtype} incl={include_self}: rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]
    assert rel_err(chained, one) <= (1e-5 if dtype == "f32" else 1e-2)
    assert rel_err(S.astype(np.float64), rS) <= S_TOL[dtype]
    assert rel_err(z.astype(np.float64), rz) <= Z_TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("qk_scale,g_scale", [(2.0 ** -10, 1.0), (32.0, 32.0)], ids=["qk_near_eps", "large"])
def test_token_causal_scaled_inputs(dtype, qk_scale, g_scale):
    """q and k scaled by powers of two (exact in bf16) down to where mean(q^2)
    meets eps, or up with the gates in the sigmoid's saturated range: the
    walk's folded normalisation (eps * rms(q) in the denominator) and gate."""
    from workloads import f32_to_bf16_bits
    inp = make_inputs(3, 6, 8, 2, 128, dtype, seed=44)
    for name, sc in (("q", qk_scale), ("k", qk_scale), ("g", g_scale)):
        inp[name] = (inp[name] * np.float32(sc)).astype(np.float32)
        if dtype == "bf16":
            inp[name + "_bits"] = f32_to_bf16_bits(inp[name])
    _check(f"tc scaled q,k x{qk_scale:g} g x{g_scale:g} {dtype}", inp, True)


def test_token_causal_first_token_strict_is_zero():
    """Strictly earlier tokens and no carried state: token 0 reads nothing and
    its output is exactly zero."""
    inp = make_inputs(2, 4, 4, 2, 64, "bf16", seed=35)
    out, _, _ = run_token_causal(to_device(inp), inp["grid"], inp["eps"], False)
    o = to_f64(out)
    assert np.all(o[0] == 0.0)
    assert np.all(np.isfinite(o))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_token_causal_one_head_kernel(plan, dtype):
    """d = 128 with the head-pair kernel switched off: the one-head walk."""
    plan("pass2_generic", 1)
    inp = make_inputs(4, 5, 9, 4, 128, dtype, seed=38)
    _check(f"tc one-head kernel {dtype}", inp, True)


def test_token_causal_global_rope_table(plan):
    plan("rope_global", 1)
    inp = make_inputs(4, 6, 7, 2, 128, "bf16", seed=36)
    _check("tc global rope", inp, True)


def test_token_causal_deterministic():
    torch = pytest.importorskip("torch")
    inp = make_inputs(3, 8, 9, 4, 128, "bf16", seed=37)
    dev = to_device(inp)
    a, Sa, za = run_token_causal(dev, inp["grid"], inp["eps"], True)
    b, Sb, zb = run_token_causal(dev, inp["grid"], inp["eps"], True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(Sa, Sb) and torch.equal(za, zb)


def test_token_causal_empty_grid_leaves_state():
    torch = pytest.importorskip("torch")
    import gated_bidirectional_linear_amd as gla
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    beta = torch.zeros((0, 2), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, device="cuda")
    S = torch.full((2, 64, 64), 1.5, device="cuda")
    z = torch.full((2, 64), 0.5, device="cuda")
    gla.token_causal_forward(q, q, q, beta, q, w, (0, 4, 4), S, z)
    torch.cuda.synchronize()
    assert bool((S == 1.5).all()) and bool((z == 0.5).all())


@pytest.mark.parametrize("eps", [float(np.finfo(np.float32).tiny), float(np.float32(1e-14))],
                         ids=["flt_min", "1e-14"])
@pytest.mark.parametrize("kernel", ["head_pair", "f32"])
@pytest.mark.parametrize("include_self", [True, False])
def test_token_causal_tiny_eps_zero_rows(include_self, kernel, eps):
    """The smallest eps the interface accepts (FLT_MIN) and 1e-14, with
    all-zero and all-negative q rows (exactly zero output), and in the strict
    reading token 0 on a fresh state (no earlier token: numerator 0,
    denominator eps * rms(q)), also exactly zero; the head-pair walk (bf16,
    d = 128) and the one-head walk (fp32)."""
    from workloads import f32_to_bf16_bits
    dtype = "f32" if kernel == "f32" else "bf16"
    d = 64 if kernel == "f32" else 128
    inp = make_inputs(4, 5, 9, 4, d, dtype, seed=45, eps=eps)
    inp["q"][5::5] = 0.0
    inp["q"][1::5] = -np.abs(inp["q"][1::5])
    inp["q"][0] = np.abs(inp["q"][0])
    if dtype == "bf16":
        inp["q_bits"] = f32_to_bf16_bits(inp["q"])
    o = _check(f"tc eps={eps:.3e} {kernel} incl={include_self}", inp, include_self)
    assert np.all(o[5::5] == 0) and np.all(o[1::5] == 0)
    if not include_self:
        assert np.all(o[0] == 0)
    else:
        assert np.any(o[0] != 0)


@pytest.mark.parametrize("include_self,dtype", [(True, "bf16"), (False, "bf16"), (True, "fp8")])
def test_token_causal_long_sequence_sampled(include_self, dtype):
    """720p/60s (N = 159,280, 32 heads) at full size in the default launch
    plan: every head at the same 2,100 tokens (every segment boundary, the
    first and last tokens and random ones) against the oracle's running sums,
    8 heads per oracle call, and the final state of every head against the
    bidirectional state."""
    torch = pytest.importorskip("torch")
    w = dataclasses.replace(WORKLOADS["720p_60s"], dtype=dtype)
    print(f"[case] token-causal {w.name} {dtype} N={w.N} heads={w.heads} include_self={include_self}", flush=True)
    inp = make_workload_inputs(w, seed=0, keep_f32=False)
    dev = to_device(inp)
    out, S, z = run_token_causal(dev, inp["grid"], inp["eps"], include_self)
    del dev
    assert bool(torch.isfinite(out.float()).all())
    # default plan: 512 workgroups -> 16 segments of 9,984 tokens per head
    seg = 9984
    bounds = [s * seg + dlt for s in range(1, 16) for dlt in (-1, 0, 1)]
    rng = np.random.default_rng(321)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, w.N - 1], bounds, rng.integers(0, w.N, 2060)]))
    assert len(rows) >= 2048

    def ref_rows(sub):
        return orc.gla_token_causal_rows(sub["q"], sub["k"], sub["v"], sub["beta"], sub["g"], sub["rms_w"],
                                         sub["grid"], sub["eps"], rows, include_self=include_self)

    err = grouped_head_error(out, inp, ref_rows, kind=dtype if dtype in ("fp8", "e5m2") else "rel", rows=rows,
                             label=f"tc 720p_60s {dtype} incl={include_self}")
    print(f"[parity] tc 720p_60s {dtype} all heads, {len(rows)} rows, incl={include_self}: error {err:.3e}",
          flush=True)
    assert err <= TOL[dtype]
    for h0 in range(0, w.heads, 8):
        hs = list(range(h0, h0 + 8))
        sub = head_slice_f32(inp, hs)
        parts = orc.gla_forward(sub["q"], sub["k"], sub["v"], sub["beta"], sub["g"], sub["rms_w"], sub["grid"],
                                sub["eps"], rows=np.array([0]), return_parts=True)
        assert rel_err(to_f64(S[hs]), parts["S"]) <= S_TOL[dtype]
        assert rel_err(to_f64(z[hs]), parts["z"]) <= Z_TOL[dtype]


@pytest.mark.parametrize("include_self", [True, False])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_causal_single_token(dtype, include_self):
    """One token: it reads the carried state (and itself when included)."""
    inp = make_inputs(1, 1, 1, 2, 128, dtype, seed=39)
    S0, z0 = make_state(2, 128, seed=5)
    _check(f"tc single token {dtype} incl={include_self}", inp, include_self, S0, z0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_causal_large_frame_offset(dtype):
    """Frames far into a sequence: RoPE positions t_offset + t against the
    oracle with the same position offset, from a carried state; the offset
    moves the oracle's output by far more than the kernel's error."""
    T, H, W, heads, t_off = 3, 5, 6, 2, 1000
    d = 64 if dtype == "f32" else 128
    inp = make_inputs(T, H, W, heads, d, dtype, seed=40)
    S0, z0 = make_state(heads, d, seed=6)
    o = _check(f"tc frame offset {t_off} {dtype}", inp, True, S0, z0, t_offset=t_off)
    ro, _, _ = _oracle_tc(inp, True, S0, z0, pos_offset=(t_off, 0, 0))
    plain, _, _ = _oracle_tc(inp, True, S0, z0)
    assert rel_err(plain, ro) > max(10 * rel_err(o, ro), TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("include_self", [True, False])
def test_token_causal_wide_frame(dtype, include_self):
    """34 x 60 latent frames (1080p): the register pass 1 stages the wide RoPE
    table (2,256 y and x entries) and the walk reads the global table."""
    import gated_bidirectional_linear_amd as gla
    code = gla.DTYPE_BF16 if dtype == "bf16" else gla.DTYPE_FP8_E4M3
    p = gla.plan_describe("token_causal", (1, 34, 60), 2, 128, code)
    assert (p["pass1_reg"], p["rope_lds1"], p["rope_lds2"]) == (1, 1, 0)
    inp = make_inputs(1, 34, 60, 2, 128, dtype, seed=41)
    S0, z0 = make_state(2, 128, seed=7)
    _check(f"tc wide frame {dtype} incl={include_self}", inp, include_self, S0, z0)
