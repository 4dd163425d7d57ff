"""GPU parity of batched calls: B independent sequences of one grid in one
launch sequence ([B, N, heads, d] tensors, per-item carried states).  Every
item is checked against the fp64 oracle on that item alone and against the
single-sequence call on the same item."""
import numpy as np
import pytest

import oracle.gla_oracle as orc
from workloads import WORKLOADS, make_inputs, make_state
from tests.gpu_helpers import (FP8_ROUNDING, TOL, Z_TOL, fp8_excess, rel_err, run_block_causal, run_forward,
                               run_token_causal, to_device, to_f64)

pytestmark = pytest.mark.gpu

S_TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2, "e5m2": 1e-2}


def _items(B, T, H, W, heads, d, dtype, seed, eps=1e-6):
    its = [make_inputs(T, H, W, heads, d, dtype, seed=seed + b, eps=eps) for b in range(B)]
    for it in its[1:]:
        it["rms_w"] = its[0]["rms_w"]     # one RMSNorm weight for the whole batch
    return its


def _stack(its):
    import torch
    devs = [to_device(it) for it in its]
    out = {n: torch.stack([dv[n] for dv in devs]).contiguous() for n in ("q", "k", "v", "g", "beta")}
    out["rms_w"] = devs[0]["rms_w"]
    return out, devs


def _err(got, ref, dtype):
    return fp8_excess(got, ref, dtype) if dtype in ("fp8", "e5m2") else rel_err(got, ref)


def _agree(got, other, dtype) -> float:
    """Difference of two GPU outputs of the same item (batched and single
    calls, whose launch plans may differ) relative to max|other|.  An fp8
    output is rounded on each side, so the two may sit one output step apart:
    twice the format's rounding bound (FP8_ROUNDING) is allowed before the
    path's own difference is counted."""
    if dtype not in ("fp8", "e5m2"):
        return rel_err(got, other)
    rel, ab = FP8_ROUNDING[dtype]
    ex = np.abs(got - other) - 2.0 * (rel * np.maximum(np.abs(got), np.abs(other)) + ab)
    den = float(np.max(np.abs(other)))
    return max(0.0, float(np.max(ex))) / (den if den > 0 else 1.0)


def _oracle(it, **kw):
    return orc.gla_forward(it["q"], it["k"], it["v"], it["beta"], it["g"], it["rms_w"], it["grid"], it["eps"], **kw)


# (B, T, H, W, heads, d, dtype): ragged token counts, odd head count (one-head kernels), every dtype
SHAPES = [
    (3, 3, 5, 7, 2, 64, "f32"),
    (3, 4, 6, 10, 4, 128, "bf16"),
    (2, 5, 9, 3, 3, 128, "bf16"),
    (3, 3, 4, 5, 2, 128, "fp8"),
    (2, 3, 4, 5, 4, 128, "e5m2"),
    (2, 2, 34, 60, 4, 128, "bf16"),   # 1080p frames: RoPE tables past 2,048 entries, per item
    (2, 2, 34, 60, 4, 128, "fp8"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_batch_forward(shape):
    import gated_bidirectional_linear_amd as gla
    import torch
    B, T, H, W, heads, d, dtype = shape
    print(f"[case] batch forward {shape}", flush=True)
    its = _items(B, T, H, W, heads, d, dtype, seed=50)
    dev, devs = _stack(its)
    out = gla.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], (T, H, W), eps=its[0]["eps"])
    torch.cuda.synchronize()
    for b, it in enumerate(its):
        got = to_f64(out[b])
        err = _err(got, _oracle(it), dtype)
        print(f"[parity] batch {shape} item {b}: {err:.3e}", flush=True)
        assert np.all(np.isfinite(got))
        assert err <= TOL[dtype]
        single = to_f64(run_forward(devs[b], it["grid"], it["eps"]))
        assert _agree(got, single, dtype) <= (1e-5 if dtype == "f32" else TOL[dtype])


def test_batch_of_one_is_the_single_call():
    """A [1, N, heads, d] call plans and computes exactly as the [N, heads, d] call."""
    import gated_bidirectional_linear_amd as gla
    import torch
    its = _items(1, 5, 9, 13, 4, 128, "bf16", seed=60)
    dev, devs = _stack(its)
    out = gla.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], (5, 9, 13))
    single = run_forward(devs[0], its[0]["grid"], its[0]["eps"])
    assert torch.equal(out[0].view(torch.int16), single.view(torch.int16))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
@pytest.mark.parametrize("t_offset", [0, 4])
def test_batch_block_causal(dtype, d, t_offset):
    """Per-item carried states; the last block of every item is shorter (T = 5,
    F = 2); a frame offset applies to every item alike."""
    import gated_bidirectional_linear_amd as gla
    import torch
    B, T, H, W, heads, F = 3, 5, 4, 6, 2, 2
    print(f"[case] batch block-causal {dtype} d={d} t_offset={t_offset}", flush=True)
    its = _items(B, T, H, W, heads, d, dtype, seed=70)
    dev, devs = _stack(its)
    states = [make_state(heads, d, seed=80 + b) for b in range(B)]
    S = torch.from_numpy(np.stack([s for s, _ in states])).cuda()
    z = torch.from_numpy(np.stack([zz for _, zz in states])).cuda()
    out = gla.block_causal_forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], (T, H, W),
                                   S, z, F, eps=its[0]["eps"], t_offset=t_offset)
    torch.cuda.synchronize()
    for b, it in enumerate(its):
        ro, rS, rz = orc.gla_block_causal_forward(it["q"], it["k"], it["v"], it["beta"], it["g"], it["rms_w"],
                                                  it["grid"], it["eps"], F, S0=states[b][0], z0=states[b][1],
                                                  pos_offset=(t_offset, 0, 0))
        err = rel_err(to_f64(out[b]), ro)
        print(f"[parity] batch block-causal {dtype} item {b}: {err:.3e}", flush=True)
        assert err <= TOL[dtype]
        assert rel_err(to_f64(S[b]), rS) <= S_TOL[dtype]
        assert rel_err(to_f64(z[b]), rz) <= Z_TOL[dtype]
        so, sS, sz = run_block_causal(devs[b], it["grid"], it["eps"], F, states[b][0], states[b][1], t_offset)
        assert rel_err(to_f64(out[b]), to_f64(so)) <= (1e-5 if dtype == "f32" else TOL[dtype])


@pytest.mark.parametrize("include_self", [True, False])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("fp8", 128)])
def test_batch_token_causal(dtype, d, include_self):
    import gated_bidirectional_linear_amd as gla
    import torch
    B, T, H, W, heads = 2, 3, 5, 7, 2
    print(f"[case] batch token-causal {dtype} d={d} include_self={include_self}", flush=True)
    its = _items(B, T, H, W, heads, d, dtype, seed=90)
    dev, devs = _stack(its)
    states = [make_state(heads, d, seed=95 + b) for b in range(B)]
    S = torch.from_numpy(np.stack([s for s, _ in states])).cuda()
    z = torch.from_numpy(np.stack([zz for _, zz in states])).cuda()
    out = gla.token_causal_forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], (T, H, W),
                                   S, z, include_self=include_self, eps=its[0]["eps"])
    torch.cuda.synchronize()
    for b, it in enumerate(its):
        ro, rS, rz = orc.gla_token_causal_forward(it["q"], it["k"], it["v"], it["beta"], it["g"], it["rms_w"],
                                                  it["grid"], it["eps"], include_self=include_self,
                                                  S0=states[b][0], z0=states[b][1])
        err = _err(to_f64(out[b]), ro, dtype)
        print(f"[parity] batch token-causal {dtype} incl={include_self} item {b}: {err:.3e}", flush=True)
        assert err <= TOL[dtype]
        assert rel_err(to_f64(S[b]), rS) <= S_TOL[dtype]
        assert rel_err(to_f64(z[b]), rz) <= Z_TOL[dtype]


def test_batch_480p():
    """Four 480p videos (4,290 tokens, 20 heads each) in one call."""
    import gated_bidirectional_linear_amd as gla
    import torch
    w = WORKLOADS["480p"]
    its = _items(4, w.T, w.H, w.W, w.heads, w.d, "bf16", seed=100, eps=w.eps)
    dev, _ = _stack(its)
    out = gla.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], (w.T, w.H, w.W), eps=w.eps)
    torch.cuda.synchronize()
    for b, it in enumerate(its):
        err = rel_err(to_f64(out[b]), _oracle(it))
        print(f"[parity] batch 480p item {b}: {err:.3e}", flush=True)
        assert err <= TOL["bf16"]
