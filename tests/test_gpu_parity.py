"""GPU parity: the HIP path (called through the C ABI) against the fp64 oracle,
element by element, on seeded inputs.

Tolerances: max|err| <= 1e-5 * max|ref| for fp32 inputs and <= 2e-2 * max|ref|
for bf16 inputs with fp32 accumulation.
"""
import numpy as np
import pytest

import oracle.gla_oracle as orc
from workloads import WORKLOADS, make_inputs, make_workload_inputs, make_state
from tests.gpu_helpers import (TOL, Z_TOL, to_device, to_f64, rel_err, run_forward, run_block_causal,
                               grouped_head_error)

pytestmark = pytest.mark.gpu


def _oracle(inp, **kw):
    return orc.gla_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"], inp["grid"],
                           inp["eps"], **kw)


def _oracle_bc(inp, F, S0=None, z0=None, **kw):
    return orc.gla_block_causal_forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"],
                                        inp["grid"], inp["eps"], F, S0=S0, z0=z0, **kw)


def _report(name, err, tol):
    print(f"[parity] {name}: rel err {err:.3e} (tol {tol:.0e})", flush=True)


# ---------------------------------------------------------------------------
# The named workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wname", ["tiny_f32", "480p", "720p_5s_h20", "720p_5s_h32"])
def test_bidirectional_workload(wname):
    w = WORKLOADS[wname]
    print(f"[case] {wname} grid={w.T}x{w.H}x{w.W} heads={w.heads} d={w.d} {w.dtype}", flush=True)
    inp = make_workload_inputs(w, seed=0)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    ref = _oracle(inp)
    err = rel_err(out, ref)
    _report(wname, err, TOL[w.dtype])
    assert np.all(np.isfinite(out))
    assert err <= TOL[w.dtype]


def test_block_causal_workload():
    w = WORKLOADS["block_causal_720p"]
    print(f"[case] {w.name} F={w.block_frames}", flush=True)
    inp = make_workload_inputs(w, seed=0)
    out, S, z = run_block_causal(to_device(inp), inp["grid"], inp["eps"], w.block_frames)
    ro, rS, rz = _oracle_bc(inp, w.block_frames)
    err = rel_err(to_f64(out), ro)
    _report(w.name, err, TOL[w.dtype])
    assert err <= TOL[w.dtype]
    assert rel_err(to_f64(S), rS) <= 1e-2
    assert rel_err(to_f64(z), rz) <= Z_TOL[w.dtype]


def test_long_sequence_workload_full():
    """720p/60s (N = 159,280, 32 heads) at full size in the default launch
    plan (the one the benchmark times): every output of every head against the
    oracle, 8 heads per oracle call; every output row is also checked for the
    RMSNorm bound mean((o/w)^2) <= 1."""
    torch = pytest.importorskip("torch")
    w = WORKLOADS["720p_60s"]
    print(f"[case] {w.name} N={w.N} heads={w.heads}", flush=True)
    inp = make_workload_inputs(w, seed=0, keep_f32=False)
    dev = to_device(inp)
    out = run_forward(dev, inp["grid"], inp["eps"])
    del dev
    o32 = out.float()
    wv = torch.from_numpy(inp["rms_w"]).cuda()[None, None, :]
    ms = ((o32 / wv) ** 2).mean(dim=-1)
    assert bool(torch.isfinite(o32).all())
    assert float(ms.max()) <= 1.0 + 2e-2
    del o32, ms
    err = grouped_head_error(out, inp, lambda sub: _oracle(sub), label=w.name)
    _report(w.name + " all heads, all rows", err, TOL["bf16"])
    assert err <= TOL["bf16"]


def test_1080p_workload_full():
    """The 1080p/121-frame latent grid (16 x 34 x 60, N = 32,640, 32 heads) at
    full size in the default plan: its y and x RoPE blocks (2,256 entries at
    d = 128) are staged in LDS beside the chunk's frames, so the register
    pass 1 and the four-head output kernel run.  Every output of every head
    against the oracle, 8 heads per oracle call."""
    import gated_bidirectional_linear_amd as gla
    w = WORKLOADS["1080p_121f"]
    p = gla.plan_describe("bidirectional", (w.T, w.H, w.W), w.heads, w.d, gla.DTYPE_BF16)
    assert (p["rope_lds1"], p["rope_lds2"], p["pass1_reg"], p["pass2_heads"]) == (1, 1, 1, 4)
    print(f"[case] {w.name} N={w.N} heads={w.heads}", flush=True)
    inp = make_workload_inputs(w, seed=0, keep_f32=False)
    dev = to_device(inp)
    out = run_forward(dev, inp["grid"], inp["eps"])
    del dev
    err = grouped_head_error(out, inp, lambda sub: _oracle(sub), label=w.name)
    _report(w.name + " all heads, all rows", err, TOL["bf16"])
    assert err <= TOL["bf16"]


# ---------------------------------------------------------------------------
# Shapes: head dims, ragged token counts, tiny grids
# ---------------------------------------------------------------------------

SHAPES = [
    # (T, H, W, heads, d)
    (2, 4, 4, 2, 32),      # 32 tokens: less than one tile
    (1, 1, 1, 3, 64),      # a single token
    (3, 5, 7, 2, 64),      # 105 tokens: ragged tail
    (5, 9, 13, 3, 128),    # 585 tokens: several tiles + tail
    (7, 3, 11, 1, 32),     # 231
    (2, 1, 1, 4, 128),     # 2 tokens
    (4, 16, 16, 2, 128),   # 1024 tokens: exact tiles
    (9, 15, 26, 2, 64),    # 3510 tokens
    (2, 5, 9, 64, 128),    # 64 heads: 16 head quads, a chunk in 16-token tiles
    (1, 3, 5, 128, 64),    # 128 heads at d = 64
    (2, 4, 7, 40, 128),    # 40 heads: 10 head quads
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(shape, dtype):
    T, H, W, heads, d = shape
    print(f"[case] shape {shape} {dtype}", flush=True)
    inp = make_inputs(T, H, W, heads, d, dtype, seed=7)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"{shape} {dtype}", err, TOL[dtype])
    assert err <= TOL[dtype]


@pytest.mark.parametrize("eps", [1e-2, 1.0])
def test_eps_values(eps):
    inp = make_inputs(3, 6, 10, 2, 64, "f32", seed=8, eps=eps)
    out = to_f64(run_forward(to_device(inp), inp["grid"], eps))
    err = rel_err(out, _oracle(inp))
    _report(f"eps={eps}", err, TOL["f32"])
    assert err <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("qk_scale,g_scale", [(2.0 ** -10, 1.0), (32.0, 32.0)], ids=["qk_near_eps", "large"])
def test_scaled_inputs(dtype, qk_scale, g_scale):
    """q and k scaled by powers of two (exact in bf16) so that mean(q^2) comes
    down to eps (2^-10: ~1e-6) or far above it, and gates scaled into the
    sigmoid's saturated range (x32): the folded q-side normalisation, whose eps
    term moves into the denominator, and the gate at the ends of their range."""
    from workloads import f32_to_bf16_bits
    inp = make_inputs(5, 9, 13, 2, 128, dtype, seed=43)
    for name, sc in (("q", qk_scale), ("k", qk_scale), ("g", g_scale)):
        inp[name] = (inp[name] * np.float32(sc)).astype(np.float32)
        if dtype == "bf16":
            inp[name + "_bits"] = f32_to_bf16_bits(inp[name])
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"scaled q,k x{qk_scale:g} g x{g_scale:g} {dtype}", err, TOL[dtype])
    assert np.all(np.isfinite(out))
    assert err <= TOL[dtype]


def test_degenerate_rows():
    """All-negative q rows give exactly zero output; zero k rows add nothing."""
    inp = make_inputs(2, 5, 9, 2, 128, "bf16", seed=9)
    inp["q"][::5] = -np.abs(inp["q"][::5])
    inp["k"][1::7] = 0.0
    from workloads import f32_to_bf16_bits
    for name in ("q", "k"):
        inp[name + "_bits"] = f32_to_bf16_bits(inp[name])
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    assert np.all(out[::5] == 0)
    err = rel_err(out, _oracle(inp))
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("eps", [float(np.finfo(np.float32).tiny), float(np.float32(1e-14))],
                         ids=["flt_min", "1e-14"])
@pytest.mark.parametrize("kernel", ["head_pair", "one_head", "f32"])
def test_tiny_eps_zero_and_negative_q_rows(plan, eps, kernel):
    """The smallest eps the interface accepts (FLT_MIN) and 1e-14, with
    all-zero and all-negative q rows: those rows have phi(q) = 0, so the
    numerator is 0 and the denominator is eps * rms(q) (as small as eps^1.5),
    and their output is exactly 0; every other row matches the oracle.  Runs
    the head-pair output kernel (bf16, d = 128), the one-head kernel and the
    fp32 path."""
    from workloads import f32_to_bf16_bits
    dtype = "f32" if kernel == "f32" else "bf16"
    d = 64 if kernel == "f32" else 128
    if kernel == "one_head":
        plan("pass2_generic", 1)
    inp = make_inputs(5, 9, 13, 4, d, dtype, seed=44, eps=eps)
    inp["q"][::5] = 0.0
    inp["q"][1::5] = -np.abs(inp["q"][1::5])
    if dtype == "bf16":
        inp["q_bits"] = f32_to_bf16_bits(inp["q"])
    out = to_f64(run_forward(to_device(inp), inp["grid"], eps))
    assert np.all(np.isfinite(out))
    assert np.all(out[::5] == 0) and np.all(out[1::5] == 0)
    err = rel_err(out, _oracle(inp))
    _report(f"eps={eps:.3e} {kernel}", err, TOL[dtype])
    assert err <= TOL[dtype]


def test_zero_beta_gives_zero():
    inp = make_inputs(2, 4, 9, 2, 64, "f32", seed=10)
    inp["beta"][:] = 0.0
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    assert np.all(out == 0)


def test_deterministic():
    torch = pytest.importorskip("torch")
    inp = make_inputs(6, 11, 13, 4, 128, "bf16", seed=11)
    dev = to_device(inp)
    a = run_forward(dev, inp["grid"], inp["eps"]).clone()
    b = run_forward(dev, inp["grid"], inp["eps"])
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_grid_is_noop():
    torch = pytest.importorskip("torch")
    inp = make_inputs(0, 4, 4, 2, 64, "bf16", seed=12)
    dev = to_device(inp)
    out = run_forward(dev, inp["grid"], inp["eps"])
    assert out.shape == (0, 2, 64)
    S0, z0 = make_state(2, 64, seed=1)
    _, S, z = run_block_causal(dev, inp["grid"], inp["eps"], 2, S0, z0)
    assert np.array_equal(S.cpu().numpy(), S0) and np.array_equal(z.cpu().numpy(), z0)


# ---------------------------------------------------------------------------
# Block-causal
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,H,W,heads,d,F", [
    (7, 3, 5, 2, 64, 2),     # last block shorter
    (5, 4, 4, 2, 32, 1),     # one frame per block
    (4, 6, 6, 3, 128, 4),    # F == T: one block
    (3, 5, 5, 2, 64, 10),    # F > T
    (9, 8, 9, 2, 128, 3),    # blocks of 216 tokens: tiles straddle nothing
])
def test_block_causal_shapes(T, H, W, heads, d, F, dtype):
    print(f"[case] block-causal {(T, H, W, heads, d, F)} {dtype}", flush=True)
    inp = make_inputs(T, H, W, heads, d, dtype, seed=13)
    out, S, z = run_block_causal(to_device(inp), inp["grid"], inp["eps"], F)
    ro, rS, rz = _oracle_bc(inp, F)
    err = rel_err(to_f64(out), ro)
    _report(f"bc {(T, H, W, heads, d, F)} {dtype}", err, TOL[dtype])
    assert err <= TOL[dtype]
    s_tol = 1e-5 if dtype == "f32" else 1e-2
    assert rel_err(to_f64(S), rS) <= s_tol
    assert rel_err(to_f64(z), rz) <= Z_TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_causal_with_prior_state(dtype):
    """The carried state comes from the oracle run over a previous chunk of
    frames; the second chunk's output must match the one-call oracle."""
    T1, T2, H, W, heads, d, F = 3, 4, 5, 6, 2, 64, 2
    full = make_inputs(T1 + T2, H, W, heads, d, dtype, seed=14)
    hw = H * W
    first = {k: (v[: T1 * hw] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in full.items()}
    first["grid"] = (T1, H, W)
    _, S0, z0 = _oracle_bc(first, F)
    second = {k: (v[T1 * hw:] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in full.items()}
    second["grid"] = (T2, H, W)
    out, S, z = run_block_causal(to_device(second), second["grid"], second["eps"], F, S0, z0)
    ro, rS, rz = _oracle_bc(second, F, S0=S0, z0=z0)
    err = rel_err(to_f64(out), ro)
    _report(f"bc prior state {dtype}", err, TOL[dtype])
    assert err <= TOL[dtype]
    assert rel_err(to_f64(z), rz) <= Z_TOL[dtype]


def _frames(inp, t0, t1, hw):
    part = {k: (v[t0 * hw: t1 * hw] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in inp.items()}
    part["grid"] = (t1 - t0,) + tuple(inp["grid"][1:])
    return part


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_streaming_chained_calls_equal_one_call(dtype):
    """A video streamed through three calls with frame offsets gives the output
    and final state of one call (and of the oracle)."""
    T, H, W, heads, d, F = 9, 6, 7, 2, 128, 3
    hw = H * W
    inp = make_inputs(T, H, W, heads, d, dtype, seed=21)
    one, S1, z1 = run_block_causal(to_device(inp), inp["grid"], inp["eps"], F)
    S, z = None, None
    outs = []
    for t0, t1 in ((0, 3), (3, 6), (6, 9)):
        part = _frames(inp, t0, t1, hw)
        o, S_t, z_t = run_block_causal(to_device(part), part["grid"], part["eps"], F, S, z, t_offset=t0)
        outs.append(to_f64(o))
        S, z = S_t.cpu().numpy(), z_t.cpu().numpy()
    chained = np.concatenate(outs)
    ro, rS, rz = _oracle_bc(inp, F)
    err = rel_err(chained, ro)
    _report(f"streamed 3 calls {dtype}", err, TOL[dtype])
    assert err <= TOL[dtype]
    # the same kernels on the same values: one call and the chain agree closely
    assert rel_err(chained, to_f64(one)) <= (1e-6 if dtype == "f32" else 1e-2)
    assert rel_err(S.astype(np.float64), to_f64(S1)) <= 1e-5
    assert rel_err(z.astype(np.float64), to_f64(z1)) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_streaming_large_frame_offset(dtype):
    """Frames far into a video: RoPE positions t_offset + t against the oracle
    with the same position offset, from a carried oracle state."""
    T, H, W, heads, F, t_off = 4, 5, 6, 2, 2, 1000
    d = 64 if dtype == "f32" else 128   # the bf16 case runs the register-accumulating pass 1
    inp = make_inputs(T, H, W, heads, d, dtype, seed=22)
    S0, z0 = make_state(heads, d, seed=3)
    out, S, z = run_block_causal(to_device(inp), inp["grid"], inp["eps"], F, S0, z0, t_offset=t_off)
    ro, rS, rz = _oracle_bc(inp, F, S0=S0, z0=z0, pos_offset=(t_off, 0, 0))
    err = rel_err(to_f64(out), ro)
    _report(f"frame offset {t_off} {dtype}", err, TOL[dtype])
    assert err <= TOL[dtype]
    assert rel_err(to_f64(S), rS) <= (1e-5 if dtype == "f32" else 1e-2)
    assert rel_err(to_f64(z), rz) <= Z_TOL[dtype]
    # the offset matters: without it the oracle's output moves by far more
    # than the kernel's error (so this test would catch an ignored offset)
    plain = _oracle_bc(inp, F, S0=S0, z0=z0)[0]
    assert rel_err(plain, ro) > max(10 * err, TOL[dtype])


def test_block_causal_final_state_equals_bidirectional_state():
    inp = make_inputs(6, 5, 7, 2, 128, "f32", seed=15)
    _, S, z = run_block_causal(to_device(inp), inp["grid"], inp["eps"], 2)
    parts = _oracle(inp, return_parts=True)
    assert rel_err(to_f64(S), parts["S"]) <= 1e-5
    assert rel_err(to_f64(z), parts["z"]) <= 1e-5


def test_block_causal_single_block_equals_bidirectional():
    torch = pytest.importorskip("torch")
    inp = make_inputs(4, 5, 6, 2, 64, "bf16", seed=16)
    dev = to_device(inp)
    a = to_f64(run_forward(dev, inp["grid"], inp["eps"]))
    b, _, _ = run_block_causal(dev, inp["grid"], inp["eps"], 4)
    assert rel_err(to_f64(b), a) <= 1e-2


# ---------------------------------------------------------------------------
# Launch-plan variants: RoPE rows from the global table instead of LDS, grids
# too large for the LDS table, and different chunk counts.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_global_rope_table_path(plan, dtype):
    plan("rope_global", 1)
    inp = make_inputs(5, 9, 13, 3, 128, dtype, seed=17)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"global rope {dtype}", err, TOL[dtype])
    assert err <= TOL[dtype]


def test_large_frame_grid_falls_back_to_global_table():
    """64x64 latent pixels per frame: the y/x RoPE blocks exceed the LDS budget."""
    inp = make_inputs(2, 64, 64, 2, 128, "bf16", seed=18)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report("64x64 frame", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("grid", [(3, 34, 60), (2, 40, 80)], ids=lambda g: "x".join(map(str, g)))
def test_wide_frame_rope_rows_in_lds(grid, dtype):
    """Frames of 34 x 60 and 40 x 80 latent pixels: y and x RoPE blocks of
    2,256 and 2,880 entries at d = 128, more than 2,048, staged in LDS in more
    than one round; bf16 runs the register pass 1 and the four-head output
    kernel on them."""
    import gated_bidirectional_linear_amd as gla
    T, H, W = grid
    code = gla.DTYPE_F32 if dtype == "f32" else gla.DTYPE_BF16
    p = gla.plan_describe("bidirectional", grid, 4, 128, code)
    assert (p["rope_lds1"], p["rope_lds2"]) == (1, 1)
    if dtype == "bf16":
        assert (p["pass1_reg"], p["pass2_heads"]) == (1, 4)
    inp = make_inputs(T, H, W, 4, 128, dtype, seed=19)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"wide frame {grid} {dtype}", err, TOL[dtype])
    assert err <= TOL[dtype]


def test_pass1_chunk_spanning_128_frames():
    """One latent pixel per frame, 8,192 frames: each register pass-1 chunk
    spans 128 frames, the most its packed frame-row offsets address."""
    import gated_bidirectional_linear_amd as gla
    p = gla.plan_describe("bidirectional", (8192, 1, 1), 4, 128, gla.DTYPE_BF16)
    assert (p["pass1_reg"], p["rope_lds1"], p["chunk1"]) == (1, 1, 128)
    inp = make_inputs(8192, 1, 1, 4, 128, "bf16", seed=20)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report("128 frames per pass-1 chunk", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("wg1,wg2", [("1", "1"), ("4096", "65536"), ("37", "300")])
def test_chunking_variants(plan, wg1, wg2):
    plan("pass1_workgroups", wg1)
    plan("pass2_workgroups", wg2)
    inp = make_inputs(7, 11, 13, 2, 64, "bf16", seed=19)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"chunking {wg1}/{wg2}", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("chunks", [2, 3, 5, 9, 17, 33, 64])
@pytest.mark.parametrize("d", [64, 128])
def test_reduce_tree_sizes(plan, chunks, d):
    """Every size of the reduce kernel's tree (it is unrolled for the power of
    two at or above the chunk count): pass 1 asked for `chunks` chunks per
    head on the 480p grid (whole 64-token tiles per chunk give 2, 3, 5, 9, 17,
    23 and 34, so trees of 2 to 64 leaves), against the oracle."""
    heads = 2
    plan("pass1_workgroups", heads * chunks)
    inp = make_inputs(11, 15, 26, heads, d, "bf16", seed=23)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"{chunks} chunks per head, d={d}", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("shape", [(5, 9, 13, 3, 128), (3, 22, 40, 2, 128), (1, 1, 1, 2, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_generic_pass1_kernel_bf16(plan, shape):
    """The LDS-staged pass-1 kernel on bf16 d=128 (the register-accumulating one is the default there)."""
    plan("pass1_generic", 1)
    T, H, W, heads, d = shape
    inp = make_inputs(T, H, W, heads, d, "bf16", seed=20)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"generic pass1 {shape}", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("shape", [(3, 22, 40, 2, 128), (4, 6, 7, 4, 128), (1, 1, 1, 2, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_one_head_output_kernel_bf16(plan, shape):
    """The one-head-per-workgroup output kernel on bf16 d=128 with an even
    head count (heads are taken in pairs by default there)."""
    plan("pass2_generic", 1)
    T, H, W, heads, d = shape
    inp = make_inputs(T, H, W, heads, d, "bf16", seed=23)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"one-head output {shape}", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("shape", [(3, 22, 40, 4, 128), (4, 6, 7, 8, 128), (2, 5, 9, 6, 128), (1, 1, 1, 4, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_head_pair_output_kernel_bf16(plan, shape):
    """The two-heads-per-workgroup output kernel (bf16, d = 128, even head
    counts; capped at two heads per workgroup where four would divide the
    head count) on several head counts and grids, down to a single token."""
    plan("pass2_heads", 2)
    T, H, W, heads, d = shape
    inp = make_inputs(T, H, W, heads, d, "bf16", seed=24)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"head-pair output {shape}", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("shape", [(3, 22, 40, 4, 128), (4, 6, 7, 8, 128), (2, 5, 9, 12, 128), (1, 1, 1, 4, 128),
                                   (5, 9, 13, 20, 128), (1, 3, 5, 8, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_head_quad_output_kernel_bf16(shape):
    """The four-heads-per-workgroup output kernel with MFMA and stream waves
    (bf16, d = 128, head counts divisible by 4) on ragged grids, down to a
    single token and to chunks shorter than one 16-token tile."""
    T, H, W, heads, d = shape
    print(f"[case] quad output {shape}", flush=True)
    inp = make_inputs(T, H, W, heads, d, "bf16", seed=25)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"head-quad output {shape}", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("wg2", ["1", "7", "300", "5000"])
def test_head_quad_chunking(plan, wg2):
    """The four-head kernel with one chunk per (quad, segment) up to chunks of a
    single 64-token tile, including chunk counts that leave some workgroups
    without tokens."""
    plan("pass2_workgroups", wg2)
    inp = make_inputs(7, 11, 13, 8, 128, "bf16", seed=26)
    out = to_f64(run_forward(to_device(inp), inp["grid"], inp["eps"]))
    err = rel_err(out, _oracle(inp))
    _report(f"quad chunking {wg2}", err, TOL["bf16"])
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("T,H,W,heads,F", [(9, 8, 9, 4, 3), (7, 3, 5, 8, 2), (5, 4, 4, 12, 1), (5, 8, 16, 4, 2)])
def test_head_quad_block_causal(T, H, W, heads, F):
    """The four-head output kernel on per-block states (one segment per block
    of frames, the last block shorter), with a prior state.  In the last case
    the one-frame last block fills one of its segment's two chunks, so a
    workgroup has no tokens."""
    inp = make_inputs(T, H, W, heads, 128, "bf16", seed=27)
    S0, z0 = make_state(heads, 128, seed=7)
    out, S, z = run_block_causal(to_device(inp), inp["grid"], inp["eps"], F, S0, z0)
    ro, rS, rz = _oracle_bc(inp, F, S0=S0, z0=z0)
    err = rel_err(to_f64(out), ro)
    _report(f"quad bc {(T, H, W, heads, F)}", err, TOL["bf16"])
    assert err <= TOL["bf16"]
    assert rel_err(to_f64(z), rz) <= Z_TOL["bf16"]


def test_head_quad_equals_pair_kernel_closely(plan):
    """The four-head kernel rounds the gate to fp16 on its way through LDS; its
    output stays within one bf16 step of the pair kernel's (same numerators)."""
    torch = pytest.importorskip("torch")
    inp = make_inputs(6, 11, 13, 8, 128, "bf16", seed=28)
    dev = to_device(inp)
    a = run_forward(dev, inp["grid"], inp["eps"]).float()
    plan("pass2_heads", 2)
    b = run_forward(dev, inp["grid"], inp["eps"]).float()
    diff = (a - b).abs()
    assert float(diff.max()) <= 2.0 ** -7 * max(1.0, float(b.abs().max()))
    assert float((diff > 0).float().mean()) < 0.2
