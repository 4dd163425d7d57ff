"""Seeded random shapes through all three forms and all four I/O dtypes
against the fp64 oracle: grid sizes from one token to frames wider than the
RoPE rows' LDS table, head counts that select every output kernel, a carried
state and a frame offset for the causal forms.  The cases are drawn once
from a fixed seed, so every run checks the same ones; each id names its case."""
import numpy as np
import pytest

import oracle.gla_oracle as orc
from workloads import make_inputs, make_state
from tests.gpu_helpers import (TOL, Z_TOL, fp8_excess, rel_err, run_block_causal, run_forward, run_token_causal,
                               to_device, to_f64)

pytestmark = pytest.mark.gpu

S_TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2, "e5m2": 1e-2}


def _cases(n=40, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        form = ["bidirectional", "block_causal", "token_causal"][int(rng.integers(3))]
        dtype = ["f32", "bf16", "fp8", "e5m2"][int(rng.integers(4))]
        d = [32, 64, 128, 128][int(rng.integers(4))]
        heads = [1, 2, 3, 4, 4, 8, 8][int(rng.integers(7))]
        T = int(rng.integers(1, 8))
        if rng.random() < 0.25:   # wide frames: y and x RoPE blocks past 2,048 entries at d = 128
            H, W = int(rng.integers(30, 45)), int(rng.integers(50, 70))
            T, d = min(T, 2), 128
        else:
            H, W = int(rng.integers(1, 20)), int(rng.integers(1, 30))
        N = T * H * W
        if form == "token_causal" and N > 1600:   # the masked oracle is quadratic in N
            continue
        if N * heads * d > 6_000_000:
            continue
        F = int(rng.integers(1, T + 2))          # block frames; F > T is one block
        include_self = bool(rng.random() < 0.5)
        carried = form != "bidirectional" and rng.random() < 0.5
        t_offset = int(rng.integers(0, 40)) if form != "bidirectional" and rng.random() < 0.5 else 0
        if form == "block_causal":   # a block-causal call starts on a block boundary
            t_offset -= t_offset % F
        out.append((form, T, H, W, heads, d, dtype, F, include_self, carried, t_offset, len(out)))
    return out


def _id(c):
    form, T, H, W, heads, d, dtype, F, inc, carried, t0, i = c
    extra = {"bidirectional": "", "block_causal": f"-F{F}", "token_causal": "-self" if inc else "-strict"}[form]
    return f"{i:02d}-{form}{extra}-{T}x{H}x{W}-h{heads}-d{d}-{dtype}" + ("-state" if carried else "") + \
        (f"-t{t0}" if t0 else "")


def _out_err(got, ref, dtype):
    return fp8_excess(got, ref, dtype) if dtype in ("fp8", "e5m2") else rel_err(got, ref)


@pytest.mark.parametrize("case", _cases(), ids=_id)
def test_random_shape(case):
    form, T, H, W, heads, d, dtype, F, include_self, carried, t_offset, i = case
    print(f"[case] {_id(case)}", flush=True)
    inp = make_inputs(T, H, W, heads, d, dtype, seed=900 + i)
    args = (inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], inp["rms_w"], inp["grid"], inp["eps"])
    S0, z0 = make_state(heads, d, seed=950 + i) if carried else (None, None)
    dev = to_device(inp)
    if form == "bidirectional":
        got = to_f64(run_forward(dev, inp["grid"], inp["eps"]))
        ref = orc.gla_forward(*args)
        S = rS = None
    elif form == "block_causal":
        out, S, z = run_block_causal(dev, inp["grid"], inp["eps"], F, S0, z0, t_offset)
        ref, rS, rz = orc.gla_block_causal_forward(*args, F, S0=S0, z0=z0, pos_offset=(t_offset, 0, 0))
        got = to_f64(out)
    else:
        out, S, z = run_token_causal(dev, inp["grid"], inp["eps"], include_self, S0, z0, t_offset)
        ref, rS, rz = orc.gla_token_causal_forward(*args, include_self=include_self, S0=S0, z0=z0,
                                                    pos_offset=(t_offset, 0, 0))
        got = to_f64(out)
    err = _out_err(got, ref, dtype)
    print(f"[parity] {_id(case)}: {err:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= TOL[dtype]
    if S is not None:
        assert rel_err(to_f64(S), rS) <= S_TOL[dtype]
        assert rel_err(to_f64(z), rz) <= Z_TOL[dtype]
