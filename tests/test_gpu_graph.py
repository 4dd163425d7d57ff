"""HIP graph capture of the operator: a call enqueued under stream capture
(its scratch taken and returned stream-ordered, no memset nodes) replays to
the eager result, several times, with eager work and synchronisations between
the replays."""
import numpy as np
import pytest

from workloads import make_inputs
from tests.gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _graph_replays(fn, out, eager_ref, reps=3):
    torch = pytest.importorskip("torch")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on the capture stream (pool, library load)
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for r in range(reps):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bits = torch.int16 if out.element_size() == 2 else (torch.uint8 if out.element_size() == 1 else torch.int32)
        assert torch.equal(out.view(bits), eager_ref.view(bits)), f"replay {r} differs"
        _ = (eager_ref.float() * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("dtype,grid", [("bf16", (4, 9, 10)), ("fp8", (4, 9, 10)), ("e5m2", (4, 9, 10)),
                                        ("bf16", (2, 34, 60))], ids=lambda x: "x".join(map(str, x))
                         if isinstance(x, tuple) else x)
def test_forward_graph_replay(dtype, grid):
    """Four heads at d = 128: the four-head output kernel (bf16 or fp8 rows);
    34 x 60 frames run the wide-table pass 1."""
    torch = pytest.importorskip("torch")
    import gated_bidirectional_linear_amd as gla
    inp = make_inputs(*grid, 4, 128, dtype, seed=51)
    dev = to_device(inp)
    ref = gla.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], inp["grid"], eps=inp["eps"])
    torch.cuda.synchronize()
    out = torch.empty_like(ref)

    def call():
        gla.forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], inp["grid"], eps=inp["eps"],
                    out=out)
    _graph_replays(call, out, ref)


def test_token_causal_graph_replay():
    """The carried state is re-initialised inside the graph by a fill kernel
    (torch's zero_), so every replay computes the same call."""
    torch = pytest.importorskip("torch")
    import gated_bidirectional_linear_amd as gla
    inp = make_inputs(3, 8, 9, 4, 128, "bf16", seed=52)
    dev = to_device(inp)
    heads, d = 4, 128
    S = torch.zeros((heads, d, d), dtype=torch.float32, device="cuda")
    z = torch.zeros((heads, d), dtype=torch.float32, device="cuda")
    ref = gla.token_causal_forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], inp["grid"],
                                   S, z, include_self=True, eps=inp["eps"])
    torch.cuda.synchronize()
    S_ref, z_ref = S.clone(), z.clone()
    out = torch.empty_like(ref)

    def call():
        S.zero_()
        z.zero_()
        gla.token_causal_forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], dev["rms_w"], inp["grid"],
                                 S, z, include_self=True, eps=inp["eps"], out=out)
    _graph_replays(call, out, ref)
    assert torch.equal(S, S_ref) and torch.equal(z, z_ref)


def test_batched_token_causal_graph_replay():
    """A batched call ([B, N, heads, d], per-item states) under capture."""
    torch = pytest.importorskip("torch")
    import gated_bidirectional_linear_amd as gla
    B, heads, d = 3, 2, 128
    items = [to_device(make_inputs(2, 6, 7, heads, d, "bf16", seed=53 + b)) for b in range(B)]
    dev = {n: torch.stack([it[n] for it in items]).contiguous() for n in ("q", "k", "v", "g", "beta")}
    rms_w = items[0]["rms_w"]
    S = torch.zeros((B, heads, d, d), dtype=torch.float32, device="cuda")
    z = torch.zeros((B, heads, d), dtype=torch.float32, device="cuda")
    ref = gla.token_causal_forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], rms_w, (2, 6, 7), S, z)
    torch.cuda.synchronize()
    S_ref, z_ref = S.clone(), z.clone()
    out = torch.empty_like(ref)

    def call():
        S.zero_()
        z.zero_()
        gla.token_causal_forward(dev["q"], dev["k"], dev["v"], dev["beta"], dev["g"], rms_w, (2, 6, 7), S, z,
                                 out=out)
    _graph_replays(call, out, ref)
    assert torch.equal(S, S_ref) and torch.equal(z, z_ref)
