"""Pins for the fp64 oracle, checked against things other than the oracle itself.

Every check here is either brute force on tiny inputs (explicit N x N
numerator/denominator matrices with explicit per-token rotation matrices), a
closed form, an invariant the mathematics fixes, or a textbook special case.
The planted-mistake tests at the bottom show that a plausible slip in the
oracle (transposed state, flipped RoPE sign, rotate-half pairing, beta in the
key sum, RoPE before ReLU, missing q/k normalisation) fails at least one pin.
"""
import math

import numpy as np
import pytest

import oracle.gla_oracle as orc
from workloads import WORKLOADS, make_inputs, make_workload_inputs

RTOL_EXACT = 1e-11


# ----------------------------------------------------------------------------
# An independent brute-force evaluation: explicit rotation matrices, explicit
# N x N kernel matrices, no factorisation.
# ----------------------------------------------------------------------------

def _rotation_matrix(t, y, x, d, base=10000.0, off=(0, 0, 0)):
    """Block-diagonal d x d rotation for one token, built channel by channel."""
    R = np.eye(d)
    widths = (d // 4, 3 * d // 8, 3 * d // 8)
    pos = (t + off[0], y + off[1], x + off[2])
    c0 = 0
    for a in range(3):
        da = widths[a]
        for i in range(da // 2):
            ang = pos[a] * base ** (-(2.0 * i) / da)
            ch = c0 + 2 * i
            R[ch, ch] = math.cos(ang)
            R[ch, ch + 1] = -math.sin(ang)
            R[ch + 1, ch] = math.sin(ang)
            R[ch + 1, ch + 1] = math.cos(ang)
        c0 += da
    return R


def brute_force(q, k, v, beta, g, w, grid, eps, rope=True, block_frames=None, S0=None, z0=None,
                off=(0, 0, 0), token_causal=None):
    """o_j = w * rmsnorm( sig(g_j) * sum_n A_jn v_n / (sum_n D_jn + eps) ), with
    A_jn = beta_n (R_j phi q_j).(R_n phi k_n), D_jn = phi q_j . phi k_n, and for the
    block-causal form the mask blk(n) <= blk(j) plus the carried state; for the
    token-causal form ("incl" or "excl") the mask n <= j or n < j."""
    T, H, W = grid
    N, nh, d = q.shape
    toks = [(t, y, x) for t in range(T) for y in range(H) for x in range(W)]
    Rs = [(_rotation_matrix(*p, d, off=off) if rope else np.eye(d)) for p in toks]
    blk = np.array([p[0] // block_frames for p in toks]) if block_frames else np.zeros(N, int)
    out = np.zeros((N, nh, d))
    nums = np.zeros((N, nh, d))
    dens = np.zeros((N, nh))
    for h in range(nh):
        qh = q[:, h, :].astype(np.float64)
        kh = k[:, h, :].astype(np.float64)
        qn = qh / np.sqrt((qh ** 2).mean(axis=1, keepdims=True) + eps)
        kn = kh / np.sqrt((kh ** 2).mean(axis=1, keepdims=True) + eps)
        pq = np.where(qn > 0, qn, 0.0)
        pk = np.where(kn > 0, kn, 0.0)
        rq = np.stack([Rs[n] @ pq[n] for n in range(N)])
        rk = np.stack([Rs[n] @ pk[n] for n in range(N)])
        A = (rq @ rk.T) * beta[:, h].astype(np.float64)[None, :]
        D = pq @ pk.T
        M = (blk[None, :] <= blk[:, None]).astype(np.float64)
        if token_causal is not None:
            n_idx = np.arange(N)
            M = ((n_idx[None, :] <= n_idx[:, None]) if token_causal == "incl"
                 else (n_idx[None, :] < n_idx[:, None])).astype(np.float64)
        num = (A * M) @ v[:, h, :].astype(np.float64)
        den = (D * M).sum(axis=1) + eps
        if S0 is not None:
            num = num + rq @ np.asarray(S0[h], np.float64).T
            den = den + pq @ np.asarray(z0[h], np.float64)
        xg = (1.0 / (1.0 + np.exp(-g[:, h, :].astype(np.float64)))) * num / den[:, None]
        o = w[None, :] * xg / np.sqrt((xg ** 2).mean(axis=1, keepdims=True) + eps)
        out[:, h, :] = o
        nums[:, h, :] = num
        dens[:, h] = den
    return out, nums, dens


def _relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _inputs(T, H, W, nh, d, seed, dtype="f32"):
    return make_inputs(T, H, W, nh, d, dtype, seed=seed)


def _args(inp):
    return (inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"], inp["grid"], inp["eps"])


# ----------------------------------------------------------------------------
# Pins of the building blocks
# ----------------------------------------------------------------------------

def test_rms_normalize_closed_form():
    d = 32
    for c in (-3.0, 0.5, 7.0):
        x = np.full((1, d), c)
        y = orc.rms_normalize(x, 1e-6)
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-14, atol=0)
    # zero row maps to zero (no NaN)
    assert np.all(orc.rms_normalize(np.zeros((2, d)), 1e-6) == 0)


def test_rope_t_axis_frequencies_at_d32():
    """d=32 splits into (8,12,12); the t slice has 4 pairs turning by
    10000^(-2i/8) = 10^(-i) per frame: 1, 0.1, 0.01, 0.001 rad at t=1."""
    d = 32
    ang = orc.rope_angles(2, 1, 1, d)      # tokens (t=0,0,0), (t=1,0,0)
    probe_angles = []
    for p in range(d // 2):
        e = np.zeros((2, d))
        e[:, 2 * p] = 1.0
        r = orc.rope_rotate(e, ang)[1]     # token t=1
        probe_angles.append(math.atan2(r[2 * p + 1], r[2 * p]))
        other = np.delete(r, [2 * p, 2 * p + 1])
        assert np.all(other == 0), "a rotation must only mix its own channel pair"
    expected = [1.0, 0.1, 0.01, 0.001] + [0.0] * 12
    assert np.allclose(probe_angles, expected, rtol=1e-13, atol=1e-15)
    # token t=0 is not rotated at all
    assert np.all(ang[0] == 0)


def test_rope_axis_split_and_sign():
    """y rotates only channels [d/4, 5d/8), x only [5d/8, d); rotating (1,0) by a
    small positive angle gives a positive second component (counter-clockwise)."""
    d = 64
    T, H, W = 1, 3, 4
    ang = orc.rope_angles(T, H, W, d)
    x = np.random.default_rng(1).standard_normal((T * H * W, d))
    r = orc.rope_rotate(x, ang)
    for n in range(T * H * W):
        yy, xx = divmod(n, W)
        moved = np.nonzero(np.abs(r[n] - x[n]) > 1e-15)[0]
        if yy == 0 and xx == 0:
            assert moved.size == 0
        if yy == 0 and xx > 0:
            assert moved.min() >= 5 * d // 8
        if xx == 0 and yy > 0:
            assert moved.min() >= d // 4 and moved.max() < 5 * d // 8
    # sign: first x pair of token (0,0,1) rotates by exactly 1 rad
    e = np.zeros((T * H * W, d))
    e[:, 5 * d // 8] = 1.0
    r = orc.rope_rotate(e, ang)[1]
    assert abs(r[5 * d // 8] - math.cos(1.0)) < 1e-15 and abs(r[5 * d // 8 + 1] - math.sin(1.0)) < 1e-15
    # y axis with d_a = 24 at d=64: pair i turns by 10000^(-i/12) per row
    e = np.zeros((T * H * W, d))
    e[:, d // 4 + 2] = 1.0                   # pair i=1 of the y slice
    r = orc.rope_rotate(e, ang)[W]           # token (0,1,0)
    assert abs(math.atan2(r[d // 4 + 3], r[d // 4 + 2]) - 10.0 ** (-1.0 / 3.0)) < 1e-14


def test_rope_is_orthogonal_and_relative():
    d = 64
    grid = (3, 4, 5)
    N = 60
    rng = np.random.default_rng(2)
    x = rng.standard_normal((N, d))
    y = rng.standard_normal((N, d))
    a0 = orc.rope_angles(*grid, d)
    a1 = orc.rope_angles(*grid, d, pos_offset=(5, -2, 7))
    rx0, ry0 = orc.rope_rotate(x, a0), orc.rope_rotate(y, a0)
    rx1, ry1 = orc.rope_rotate(x, a1), orc.rope_rotate(y, a1)
    assert np.allclose(np.linalg.norm(rx0, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # all pairwise dot products depend only on position differences
    assert np.allclose(rx0 @ ry0.T, rx1 @ ry1.T, rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------------------
# Brute force vs the factorised oracle
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid,nh,d,seed", [
    ((2, 4, 4), 2, 32, 0),      # the tiny fp32 workload's shape
    ((3, 5, 7), 2, 64, 3),
    ((4, 6, 9), 1, 128, 4),     # N = 216
    ((1, 1, 1), 2, 16, 5),
    ((5, 1, 3), 3, 48, 6),
])
def test_factorised_matches_brute_force(grid, nh, d, seed):
    inp = _inputs(*grid, nh, d, seed)
    parts = orc.gla_forward(*_args(inp), return_parts=True)
    bo, bn, bd = brute_force(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                             inp["rms_w"].astype(np.float64), grid, inp["eps"])
    assert _relerr(parts["num"], bn) < RTOL_EXACT
    assert _relerr(parts["den"], bd) < RTOL_EXACT
    assert _relerr(parts["out"], bo) < RTOL_EXACT


def test_tiny_workload_matches_brute_force():
    w = WORKLOADS["tiny_f32"]
    inp = make_workload_inputs(w, seed=0)
    o = orc.gla_forward(*_args(inp))
    bo, _, _ = brute_force(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                           inp["rms_w"].astype(np.float64), inp["grid"], inp["eps"])
    assert _relerr(o, bo) < RTOL_EXACT


@pytest.mark.parametrize("eps", [1e-6, 1e-2, 1.0])
def test_eps_sweep_matches_brute_force(eps):
    grid = (2, 3, 5)
    inp = _inputs(*grid, 2, 32, 11)
    args = list(_args(inp))
    args[-1] = eps
    o = orc.gla_forward(*args)
    bo, _, _ = brute_force(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                           inp["rms_w"].astype(np.float64), grid, eps)
    assert _relerr(o, bo) < RTOL_EXACT


def test_associativity_of_state():
    """(RQ RK^T)(beta v) == RQ ((beta v)^T RK)^T on the oracle's own features."""
    inp = _inputs(3, 4, 5, 1, 64, 9)
    parts = orc.gla_forward(*_args(inp), return_parts=True)
    ang = orc.rope_angles(3, 4, 5, 64)
    _, rk = orc.head_features(inp["k"][:, 0, :].astype(np.float64), ang, inp["eps"])
    _, rq = orc.head_features(inp["q"][:, 0, :].astype(np.float64), ang, inp["eps"])
    bv = inp["beta"][:, 0:1].astype(np.float64) * inp["v"][:, 0, :]
    quad = (rq @ rk.T) @ bv
    assert _relerr(parts["num"][:, 0, :], quad) < RTOL_EXACT


# ----------------------------------------------------------------------------
# Closed forms and invariants
# ----------------------------------------------------------------------------

def test_single_token_closed_form():
    """N=1: the rotations cancel (R^T R = I), so with a = phi q . phi k,
    x = sig(g) * beta v a / (a + eps) and o = w * rmsnorm(x)."""
    inp = _inputs(1, 1, 1, 3, 32, 21)
    eps = inp["eps"]
    o = orc.gla_forward(*_args(inp))
    for h in range(3):
        q = inp["q"][0, h].astype(np.float64)
        k = inp["k"][0, h].astype(np.float64)
        pq = np.maximum(q / math.sqrt(np.mean(q * q) + eps), 0)
        pk = np.maximum(k / math.sqrt(np.mean(k * k) + eps), 0)
        a = float(pq @ pk)
        x = (1 / (1 + np.exp(-inp["g"][0, h].astype(np.float64)))) * inp["beta"][0, h] * inp["v"][0, h] * a / (a + eps)
        ref = inp["rms_w"] * x / math.sqrt(np.mean(x * x) + eps)
        assert _relerr(o[0, h], ref) < 1e-12


def test_single_token_at_nonzero_position():
    """Same closed form for a lone token far from the origin (rotation cancels)."""
    inp = _inputs(1, 1, 1, 2, 64, 22)
    eps = inp["eps"]
    o0 = orc.gla_forward(*_args(inp))
    o1 = orc.gla_forward(*_args(inp), pos_offset=(37, 5, 11))
    assert _relerr(o1, o0) < 1e-12


def test_zero_beta_gives_zero_output():
    inp = _inputs(2, 3, 4, 2, 32, 23)
    inp["beta"][:] = 0
    o = orc.gla_forward(*_args(inp))
    assert np.all(o == 0)


def test_identical_keys_closed_form():
    """RoPE off, every key equal: num_j = a_j sum_n beta_n v_n, den_j = N a_j + eps."""
    grid = (2, 3, 4)
    N = 24
    inp = _inputs(*grid, 2, 32, 24)
    inp["k"][:] = inp["k"][0:1]
    eps = inp["eps"]
    parts = orc.gla_forward(*_args(inp), rope=False, return_parts=True)
    for h in range(2):
        k = inp["k"][0, h].astype(np.float64)
        pk = np.maximum(k / math.sqrt(np.mean(k * k) + eps), 0)
        q = inp["q"][:, h].astype(np.float64)
        pq = np.maximum(q / np.sqrt(np.mean(q * q, axis=1, keepdims=True) + eps), 0)
        a = pq @ pk
        sbv = (inp["beta"][:, h:h + 1].astype(np.float64) * inp["v"][:, h]).sum(axis=0)
        assert _relerr(parts["num"][:, h], a[:, None] * sbv[None, :]) < RTOL_EXACT
        assert _relerr(parts["den"][:, h], N * a + eps) < RTOL_EXACT


def test_permutation_equivariance_without_rope():
    grid = (2, 4, 5)
    inp = _inputs(*grid, 2, 32, 25)
    o = orc.gla_forward(*_args(inp), rope=False)
    perm = np.random.default_rng(0).permutation(40)
    pinp = dict(inp)
    for name in ("q", "k", "v", "g", "beta"):
        pinp[name] = inp[name][perm]
    op = orc.gla_forward(*_args(pinp), rope=False)
    assert _relerr(op, o[perm]) < RTOL_EXACT


def test_position_shift_invariance_with_rope():
    """Shifting every position by a constant leaves all outputs unchanged."""
    inp = _inputs(3, 4, 5, 2, 64, 26)
    o0 = orc.gla_forward(*_args(inp))
    o1 = orc.gla_forward(*_args(inp), pos_offset=(4, 9, -3))
    assert _relerr(o1, o0) < 1e-10


def test_qk_scale_invariance():
    inp = _inputs(2, 3, 4, 2, 32, 27)
    args = list(_args(inp))
    args[-1] = 1e-14
    o = orc.gla_forward(*args)
    sc = dict(inp)
    sc["q"] = inp["q"] * 4.0          # powers of two keep the fp32 inputs exact
    sc["k"] = inp["k"] * 0.25
    args2 = list(_args(sc))
    args2[-1] = 1e-14
    o2 = orc.gla_forward(*args2)
    assert _relerr(o2, o) < 1e-10


def test_beta_scales_numerator_not_denominator():
    inp = _inputs(2, 3, 4, 2, 32, 28)
    p1 = orc.gla_forward(*_args(inp), return_parts=True)
    sc = dict(inp)
    sc["beta"] = inp["beta"] * 2.0
    p2 = orc.gla_forward(*_args(sc), return_parts=True)
    assert _relerr(p2["num"], 2.0 * p1["num"]) < RTOL_EXACT
    assert _relerr(p2["den"], p1["den"]) < RTOL_EXACT


def test_denominator_positive_and_output_rms():
    inp = _inputs(3, 4, 5, 2, 32, 29)
    inp["q"][::3] = -np.abs(inp["q"][::3])   # rows whose phi(q) is all zero
    inp["rms_w"][:] = 1.0
    p = orc.gla_forward(*_args(inp), return_parts=True)
    assert np.all(p["den"] >= inp["eps"])
    assert np.all(p["out"][::3] == 0)
    # with w = 1: mean(o^2) = m / (m + eps), m = mean(x^2)
    m = np.mean(p["x"] ** 2, axis=-1)
    mo = np.mean(p["out"] ** 2, axis=-1)
    assert np.allclose(mo, m / (m + inp["eps"]), rtol=1e-12)


def test_zero_rows_give_zero_and_no_nan():
    inp = _inputs(2, 2, 3, 2, 32, 30)
    inp["q"][0] = 0
    inp["k"][1] = 0
    o = orc.gla_forward(*_args(inp))
    assert np.all(np.isfinite(o))
    assert np.all(o[0] == 0)


# ----------------------------------------------------------------------------
# Block-causal pins
# ----------------------------------------------------------------------------

def _bc(inp, F, S0=None, z0=None, **kw):
    return orc.gla_block_causal_forward(*_args(inp), F, S0=S0, z0=z0, **kw)


@pytest.mark.parametrize("grid,F", [((5, 2, 3), 2), ((4, 3, 3), 1), ((6, 2, 2), 4), ((3, 2, 2), 3)])
def test_block_causal_matches_masked_brute_force(grid, F):
    inp = _inputs(*grid, 2, 32, 31)
    o, S, z = _bc(inp, F)
    bo, _, _ = brute_force(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                           inp["rms_w"].astype(np.float64), grid, inp["eps"], block_frames=F)
    assert _relerr(o, bo) < RTOL_EXACT


def test_block_causal_with_initial_state_matches_brute_force():
    grid = (4, 2, 3)
    inp = _inputs(*grid, 2, 32, 32)
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((2, 32, 32)) * 3
    z0 = np.abs(rng.standard_normal((2, 32))) * 5
    o, S, z = _bc(inp, 2, S0, z0)
    bo, _, _ = brute_force(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                           inp["rms_w"].astype(np.float64), grid, inp["eps"], block_frames=2, S0=S0, z0=z0)
    assert _relerr(o, bo) < RTOL_EXACT


def test_block_causal_invariants():
    grid = (7, 3, 4)
    inp = _inputs(*grid, 2, 64, 33)
    bi = orc.gla_forward(*_args(inp), return_parts=True)
    o, S, z = _bc(inp, 3)
    last = slice(6 * 12, 7 * 12)
    assert _relerr(o[last], bi["out"][last]) < RTOL_EXACT       # last block sees everything
    assert _relerr(S, bi["S"]) < RTOL_EXACT and _relerr(z, bi["z"]) < RTOL_EXACT
    o_all, _, _ = _bc(inp, 7)                                    # F >= T: one block
    assert _relerr(o_all, bi["out"]) < RTOL_EXACT
    o_big, _, _ = _bc(inp, 100)
    assert _relerr(o_big, bi["out"]) < RTOL_EXACT


def test_block_causal_chained_calls_equal_one_call():
    """Carrying (S, z) across two calls (second call's frames offset in time)
    reproduces one call: the constant-memory cache is exact."""
    grid = (6, 2, 3)
    inp = _inputs(*grid, 2, 32, 34)
    o, S, z = _bc(inp, 2)
    hw = 6
    a = {k: (v[: 4 * hw] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in inp.items()}
    b = {k: (v[4 * hw:] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in inp.items()}
    a["grid"] = (4, 2, 3)
    b["grid"] = (2, 2, 3)
    oa, Sa, za = _bc(a, 2)
    ob, Sb, zb = _bc(b, 2, Sa, za, pos_offset=(4, 0, 0))
    assert _relerr(np.concatenate([oa, ob]), o) < RTOL_EXACT
    assert _relerr(Sb, S) < RTOL_EXACT and _relerr(zb, z) < RTOL_EXACT


def test_state_memory_is_constant():
    """The carried state has heads*(d*d + d) entries whatever the length."""
    for T in (1, 4, 9):
        inp = _inputs(T, 2, 2, 2, 32, 35)
        _, S, z = _bc(inp, 2)
        assert S.size + z.size == 2 * (32 * 32 + 32)


def test_empty_grid():
    inp = _inputs(0, 2, 2, 2, 32, 36)
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((2, 32, 32))
    z0 = np.abs(rng.standard_normal((2, 32)))
    o, S, z = _bc(inp, 2, S0, z0)
    assert o.shape == (0, 2, 32)
    assert np.array_equal(S, S0) and np.array_equal(z, z0)


# ----------------------------------------------------------------------------
# Planted mistakes: each must trip at least one pin
# ----------------------------------------------------------------------------

def _pins_pass(monkeypatch_ctx=None):
    """Run a compact set of pins; True when all pass."""
    ok = True
    for grid, nh, d, seed in [((2, 4, 4), 2, 32, 0), ((3, 2, 5), 1, 64, 1)]:
        inp = _inputs(*grid, nh, d, seed)
        try:
            bo, _, _ = brute_force(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                                   inp["rms_w"].astype(np.float64), grid, inp["eps"])
            o = orc.gla_forward(*_args(inp))
            ok &= _relerr(o, bo) < RTOL_EXACT
            o1 = orc.gla_forward(*_args(inp), pos_offset=(3, 1, 2))
            ok &= _relerr(o1, o) < 1e-10
        except Exception:
            return False
    return bool(ok)


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


def _mut_transpose_state(monkeypatch):
    real = orc._output_rows

    def bad(pq, rq, S, z, gh, w, eps):
        return real(pq, rq, S.T, z, gh, w, eps)
    monkeypatch.setattr(orc, "_output_rows", bad)


def _mut_rope_sign(monkeypatch):
    real = orc.rope_rotate
    monkeypatch.setattr(orc, "rope_rotate", lambda x, a: real(x, -a))


def _mut_rotate_half(monkeypatch):
    def bad(x, a):
        x = np.asarray(x, np.float64)
        h = x.shape[-1] // 2
        u, w = x[..., :h], x[..., h:]
        c, s = np.cos(a), np.sin(a)
        return np.concatenate([u * c - w * s, u * s + w * c], axis=-1)
    monkeypatch.setattr(orc, "rope_rotate", bad)


def _mut_relu_after_rope(monkeypatch):
    def bad(xh, angles, eps):
        xn = orc.rms_normalize(xh, eps)
        p = orc.relu(xn)
        r = p if angles is None else orc.relu(orc.rope_rotate(xn, angles))
        return p, r
    monkeypatch.setattr(orc, "head_features", bad)


def _mut_no_qk_norm(monkeypatch):
    def bad(xh, angles, eps):
        p = orc.relu(np.asarray(xh, np.float64))
        r = p if angles is None else orc.rope_rotate(p, angles)
        return p, r
    monkeypatch.setattr(orc, "head_features", bad)


def _mut_rope_in_denominator(monkeypatch):
    real = orc._output_rows

    def bad(pq, rq, S, z, gh, w, eps):
        return real(rq, rq, S, z, gh, w, eps)
    monkeypatch.setattr(orc, "_output_rows", bad)


def _mut_axis_frequency(monkeypatch):
    real = orc.rope_angles

    def bad(T, H, W, d, base=orc.ROPE_BASE, pos_offset=(0, 0, 0)):
        return real(T, H, W, d, base=base * 10, pos_offset=pos_offset)
    monkeypatch.setattr(orc, "rope_angles", bad)


@pytest.mark.parametrize("mutant", [_mut_transpose_state, _mut_rope_sign, _mut_rotate_half,
                                    _mut_relu_after_rope, _mut_no_qk_norm, _mut_rope_in_denominator,
                                    _mut_axis_frequency])
def test_planted_mistake_is_caught(monkeypatch, mutant):
    mutant(monkeypatch)
    assert not _pins_pass()


def _mut_beta_in_key_sum(monkeypatch):
    def bad(beta_h, v_h, pk, rk):
        b = np.asarray(beta_h, dtype=np.float64)[:, None]
        return (b * v_h).T @ rk, (b * pk).sum(axis=0)
    monkeypatch.setattr(orc, "_state", bad)


def _mut_dropped_beta(monkeypatch):
    def bad(beta_h, v_h, pk, rk):
        return v_h.T @ rk, pk.sum(axis=0)
    monkeypatch.setattr(orc, "_state", bad)


@pytest.mark.parametrize("mutant", [_mut_beta_in_key_sum, _mut_dropped_beta])
def test_planted_state_mistake_is_caught(monkeypatch, mutant):
    mutant(monkeypatch)
    assert not _pins_pass()


# ----------------------------------------------------------------------------
# Token-causal pins
# ----------------------------------------------------------------------------

def _tc(inp, include_self=True, S0=None, z0=None, **kw):
    return orc.gla_token_causal_forward(*_args(inp), include_self=include_self, S0=S0, z0=z0, **kw)


@pytest.mark.parametrize("include_self", [True, False])
@pytest.mark.parametrize("grid", [(3, 2, 3), (2, 3, 2), (4, 1, 1)])
def test_token_causal_matches_masked_brute_force(grid, include_self):
    inp = _inputs(*grid, 2, 32, 51)
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((2, 32, 32))
    z0 = np.abs(rng.standard_normal((2, 32)))
    for s0, z0_ in ((None, None), (S0, z0)):
        o, S, z = _tc(inp, include_self, s0, z0_, pos_offset=(3, 0, 0))
        bo, _, _ = brute_force(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"],
                               inp["rms_w"].astype(np.float64), grid, inp["eps"], S0=s0, z0=z0_,
                               off=(3, 0, 0), token_causal="incl" if include_self else "excl")
        assert _relerr(o, bo) < RTOL_EXACT


def test_token_causal_one_token_frames_equal_block_causal():
    """On a T x 1 x 1 grid every frame is one token: the inclusive token-causal
    form is the block-causal form with one frame per block."""
    inp = _inputs(9, 1, 1, 2, 32, 52)
    o, S, z = _tc(inp, True)
    ob, Sb, zb = _bc(inp, 1)
    assert _relerr(o, ob) < RTOL_EXACT
    assert _relerr(S, Sb) < RTOL_EXACT and _relerr(z, zb) < RTOL_EXACT
    oe, _, _ = _tc(inp, False)        # the strict reading differs
    assert _relerr(oe, ob) > 1e-3


def test_token_causal_last_token_reads_everything():
    """With the own token included, the last token sees the whole sequence:
    its output is the bidirectional output there; the final state is the
    bidirectional state."""
    inp = _inputs(3, 2, 4, 2, 32, 53)
    o, S, z = _tc(inp, True)
    parts = orc.gla_forward(*_args(inp), return_parts=True)
    assert _relerr(o[-1], parts["out"][-1]) < RTOL_EXACT
    assert _relerr(S, parts["S"]) < RTOL_EXACT and _relerr(z, parts["z"]) < RTOL_EXACT


def test_token_causal_first_token_strict_reads_nothing():
    """Strictly earlier tokens only: token 0 has no numerator and den = eps, so
    its output is exactly zero (with no carried state)."""
    inp = _inputs(2, 2, 3, 2, 32, 54)
    o, _, _ = _tc(inp, False)
    assert np.all(o[0] == 0.0)
    assert np.any(o[1] != 0.0)


def test_token_causal_strict_is_inclusive_minus_own_term():
    inp = _inputs(2, 3, 3, 2, 32, 55)
    pi = _tc(inp, True, return_parts=True)
    ps = _tc(inp, False, return_parts=True)
    ang = orc.rope_angles(*inp["grid"], 32)
    for h in range(2):
        pk, rk = orc.head_features(np.asarray(inp["k"][:, h], np.float64), ang, inp["eps"])
        pq, rq = orc.head_features(np.asarray(inp["q"][:, h], np.float64), ang, inp["eps"])
        own = (np.sum(rq * rk, axis=1) * inp["beta"][:, h])[:, None] * inp["v"][:, h]
        assert _relerr(pi["num"][:, h] - own, ps["num"][:, h]) < RTOL_EXACT
        assert _relerr(pi["den"][:, h] - np.sum(pq * pk, axis=1), ps["den"][:, h]) < RTOL_EXACT


@pytest.mark.parametrize("include_self", [True, False])
def test_token_causal_chained_calls_equal_one_call(include_self):
    grid = (5, 2, 3)
    inp = _inputs(*grid, 2, 32, 56)
    o, S, z = _tc(inp, include_self)
    hw = 6
    a = {k: (v[: 2 * hw] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in inp.items()}
    b = {k: (v[2 * hw:] if isinstance(v, np.ndarray) and v.ndim >= 2 else v) for k, v in inp.items()}
    a["grid"] = (2, 2, 3)
    b["grid"] = (3, 2, 3)
    oa, Sa, za = _tc(a, include_self)
    ob, Sb, zb = _tc(b, include_self, Sa, za, pos_offset=(2, 0, 0))
    assert _relerr(np.concatenate([oa, ob]), o) < RTOL_EXACT
    assert _relerr(Sb, S) < RTOL_EXACT and _relerr(zb, z) < RTOL_EXACT


@pytest.mark.parametrize("include_self", [True, False])
def test_token_causal_rows_match_brute_force(include_self):
    """The running-sum evaluation at chosen tokens (for long sequences) agrees
    with the explicit N x N masked brute force, rows given out of order and
    repeated, with a carried state."""
    grid = (3, 3, 4)
    inp = _inputs(*grid, 2, 32, 57)
    rng = np.random.default_rng(6)
    S0 = rng.standard_normal((2, 32, 32))
    z0 = np.abs(rng.standard_normal((2, 32)))
    rows = np.array([35, 0, 17, 17, 1, 20, 34])
    got = orc.gla_token_causal_rows(*_args(inp), rows, heads=[1, 0], include_self=include_self, S0=S0, z0=z0,
                                    pos_offset=(2, 0, 0))
    bo, _, _ = brute_force(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"].astype(np.float64),
                           grid, inp["eps"], S0=S0, z0=z0, off=(2, 0, 0),
                           token_causal="incl" if include_self else "excl")
    assert _relerr(got, bo[rows][:, [1, 0]]) < RTOL_EXACT
