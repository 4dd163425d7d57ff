"""The launch planner, checked on the CPU through gla_plan_describe: every plan
covers its sequence exactly with whole tiles, keeps within the kernels'
limits (64 chunk partials per segment reduced by one tree, 64-token staged
tiles, 16-token tiles of the four-head output kernel, 32-token steps of the
token-causal walk), picks the multi-head kernels only where their shape
conditions hold, and honours the knobs.  The workload plans whose timings
the planner's constants were tuned on are pinned as well."""
import itertools

import pytest

import gated_bidirectional_linear_amd as gla
from workloads import WORKLOADS

DTYPES = (gla.DTYPE_F32, gla.DTYPE_BF16, gla.DTYPE_FP8_E4M3, gla.DTYPE_FP8_E5M2)
MAX_CHUNKS = 64
TILE = 64
QUAD_TILE = 16
TOKEN_TILE = 32
QUAD_SLOTS = 256
ROPE_LDS_ENTRIES = 3072


def _ceil(a, b):
    return -(-a // b)


def _check(form, grid, heads, d, dtype, batch=1, block_frames=1, default=True):
    T, H, W = grid
    p = gla.plan_describe(form, grid, heads, d, dtype, batch=batch, block_frames=block_frames)
    n_item = T * H * W
    L = p["seg_len"]
    # segments cover one batch item exactly
    assert L >= 1 and p["segs_item"] == _ceil(n_item, L)
    if form == "block_causal":
        F = block_frames if block_frames < T else T
        assert L == F * H * W
    if form == "bidirectional":
        assert L == n_item and p["segs_item"] == 1
    # pass 1: whole staged tiles, at most one tree of partials, no empty chunk
    assert 1 <= p["cps1"] <= MAX_CHUNKS
    assert p["chunk1"] % TILE == 0
    assert p["cps1"] * p["chunk1"] >= L > (p["cps1"] - 1) * p["chunk1"]
    # pass 2
    assert p["cps2"] >= 1
    assert p["cps2"] * p["chunk2"] >= L > (p["cps2"] - 1) * p["chunk2"]
    narrow = dtype != gla.DTYPE_F32
    if form == "token_causal":
        assert L % TOKEN_TILE == 0
        assert p["cps2"] == 1 and p["chunk2"] == L
        assert p["pass2_heads"] in (0, 2)
        if p["pass2_heads"] == 2:
            assert narrow and d == 128 and heads % 2 == 0
    else:
        assert p["pass2_heads"] in (0, 2, 4)
        if p["pass2_heads"] == 4:
            assert narrow and d == 128 and heads % 4 == 0 and p["rope_lds2"] == 1
            assert p["chunk2"] % QUAD_TILE == 0
            units = heads // 4 * p["segs_item"] * batch
            # one round of workgroups, one per CU, unless chunks had to be cut
            # further to fit their RoPE rows in LDS
            if default and (H + W) * 3 * d // 16 + T * d // 8 <= ROPE_LDS_ENTRIES:
                assert units * p["cps2"] <= max(QUAD_SLOTS, units)
        else:
            assert p["chunk2"] % TILE == 0
        if p["pass2_heads"] == 2:
            assert dtype == gla.DTYPE_BF16 and d == 128 and heads % 2 == 0 and p["rope_lds2"] == 1
    # the register-accumulating pass 1 takes narrow rows at d = 128 with RoPE rows in LDS
    if p["pass1_reg"]:
        assert narrow and d == 128 and p["rope_lds1"] == 1
    if default:   # no knob set: the fast kernels wherever their conditions hold
        assert p["pass1_reg"] == int(narrow and d == 128 and p["rope_lds1"] == 1)
        if form != "token_causal":
            assert (p["pass2_heads"] == 4) == (narrow and d == 128 and heads % 4 == 0 and p["rope_lds2"] == 1)
    return p


GRIDS = [(1, 1, 1), (2, 4, 4), (3, 5, 7), (5, 9, 13), (11, 15, 26), (16, 22, 40), (24, 22, 40), (181, 22, 40),
         (2, 64, 64), (1, 1, 1000), (7, 3, 1)]


@pytest.mark.parametrize("grid", GRIDS, ids=lambda g: "x".join(map(str, g)))
@pytest.mark.parametrize("form", ["bidirectional", "block_causal", "token_causal"])
def test_plan_invariants(form, grid):
    for heads, d, dtype, batch in itertools.product((1, 2, 3, 4, 8, 20, 32), (32, 64, 128), DTYPES, (1, 3)):
        for F in ((1, 2, 3) if form == "block_causal" else (1,)):
            _check(form, grid, heads, d, dtype, batch=batch, block_frames=F)


def test_workload_plans():
    """The plans the bench lines and the full-size parity tests run: one
    round of 256 workgroups in both passes at 720p/60s, 225 workgroups of 96
    tokens at 480p, 220 of 320 tokens at 720p/5s with 20 heads."""
    w = WORKLOADS["720p_60s"]
    for dtype in (gla.DTYPE_BF16, gla.DTYPE_FP8_E4M3, gla.DTYPE_FP8_E5M2):
        p = _check("bidirectional", (w.T, w.H, w.W), w.heads, w.d, dtype)
        assert (p["cps1"], p["chunk1"], p["pass1_reg"]) == (8, 19968, 1)
        assert (p["cps2"], p["chunk2"], p["pass2_heads"]) == (32, 4992, 4)
    w = WORKLOADS["480p"]
    p = _check("bidirectional", (w.T, w.H, w.W), w.heads, w.d, gla.DTYPE_BF16)
    assert (p["cps1"], p["chunk1"], p["cps2"], p["chunk2"], p["pass2_heads"]) == (12, 384, 45, 96, 4)
    w = WORKLOADS["720p_5s_h20"]
    p = _check("bidirectional", (w.T, w.H, w.W), w.heads, w.d, gla.DTYPE_BF16)
    assert (p["cps2"], p["chunk2"], p["pass2_heads"]) == (44, 320, 4)
    # 1080p/121 frames: the y and x RoPE blocks (2,256 entries) fit in LDS
    # beside the chunk's frames, so the register pass 1 and the four-head
    # output kernel run, one round of 256 workgroups each
    w = WORKLOADS["1080p_121f"]
    p = _check("bidirectional", (w.T, w.H, w.W), w.heads, w.d, gla.DTYPE_BF16)
    assert (p["cps1"], p["chunk1"], p["pass1_reg"], p["rope_lds1"]) == (8, 4096, 1, 1)
    assert (p["cps2"], p["chunk2"], p["pass2_heads"], p["rope_lds2"]) == (32, 1024, 4, 1)
    # one pixel per frame: register pass-1 chunks of at most 128 frames (the
    # reach of its packed frame-row offsets), else the generic kernel
    p = _check("bidirectional", (8192, 1, 1), 4, 128, gla.DTYPE_BF16)
    assert (p["pass1_reg"], p["rope_lds1"], p["chunk1"]) == (1, 1, 128)
    p = _check("bidirectional", (20000, 1, 1), 32, 128, gla.DTYPE_BF16)
    assert (p["pass1_reg"], p["rope_lds1"]) == (0, 0)
    w = WORKLOADS["block_causal_720p"]
    p = _check("block_causal", (w.T, w.H, w.W), w.heads, w.d, gla.DTYPE_BF16, block_frames=w.block_frames)
    assert (p["seg_len"], p["segs_item"], p["pass2_heads"]) == (3 * 22 * 40, 8, 4)
    p = _check("token_causal", (181, 22, 40), 32, 128, gla.DTYPE_BF16)
    assert (p["seg_len"], p["segs_item"], p["pass2_heads"]) == (9984, 16, 2)
    # y and x RoPE blocks too wide for LDS (64 + 64 positions at d = 128): the
    # global table, with chunks sized for occupancy rather than cut to the
    # smallest in search of an LDS fit
    p = _check("bidirectional", (2, 64, 64), 32, 128, gla.DTYPE_BF16)
    assert (p["rope_lds1"], p["rope_lds2"], p["pass1_reg"], p["pass2_heads"]) == (0, 0, 0, 0)
    assert p["cps1"] * 32 == 512 and p["chunk2"] > TILE
    # f32 rows: the generic kernels
    p = _check("bidirectional", (2, 4, 4), 2, 32, gla.DTYPE_F32)
    assert (p["pass1_reg"], p["pass2_heads"]) == (0, 0)


def test_knobs_steer_the_plan(plan):
    grid, heads = (16, 22, 40), 32
    base = _check("bidirectional", grid, heads, 128, gla.DTYPE_BF16)
    assert base["pass2_heads"] == 4 and base["pass1_reg"] == 1
    knob = dict(default=False)
    plan("pass2_heads", 2)
    assert _check("bidirectional", grid, heads, 128, gla.DTYPE_BF16, **knob)["pass2_heads"] == 2
    # fp8 rows have no paired-head output kernel: one head per workgroup
    assert _check("bidirectional", grid, heads, 128, gla.DTYPE_FP8_E4M3, **knob)["pass2_heads"] == 0
    plan("pass2_heads", 1)
    assert _check("bidirectional", grid, heads, 128, gla.DTYPE_BF16, **knob)["pass2_heads"] == 0
    assert _check("token_causal", grid, heads, 128, gla.DTYPE_BF16, **knob)["pass2_heads"] == 0
    gla.plan_reset()
    plan("pass2_generic", 1)
    assert _check("bidirectional", grid, heads, 128, gla.DTYPE_BF16, **knob)["pass2_heads"] == 0
    gla.plan_reset()
    plan("pass1_generic", 1)
    assert _check("bidirectional", grid, heads, 128, gla.DTYPE_BF16, **knob)["pass1_reg"] == 0
    gla.plan_reset()
    plan("rope_global", 1)
    p = _check("bidirectional", grid, heads, 128, gla.DTYPE_BF16, **knob)
    assert (p["rope_lds1"], p["rope_lds2"], p["pass1_reg"], p["pass2_heads"]) == (0, 0, 0, 0)
    gla.plan_reset()
    plan("pass1_workgroups", 64)
    assert _check("bidirectional", grid, heads, 128, gla.DTYPE_BF16, **knob)["cps1"] == 2
    gla.plan_reset()
    plan("pass2_workgroups", 1024)
    p = _check("bidirectional", grid, heads, 128, gla.DTYPE_BF16, default=False)
    L = p["seg_len"]   # 1024 / 8 units = 128 chunks, rounded to whole 64-token tiles
    assert p["chunk2"] == _ceil(_ceil(L, TILE), 128) * TILE and p["cps2"] == _ceil(L, p["chunk2"])
    gla.plan_reset()
    plan("token_causal_workgroups", 32)
    assert _check("token_causal", grid, heads, 128, gla.DTYPE_BF16, **knob)["segs_item"] == 1
    gla.plan_reset()
    assert _check("bidirectional", grid, heads, 128, gla.DTYPE_BF16) == base


def test_plan_describe_errors():
    lib = gla.load()
    import ctypes
    out = (ctypes.c_int * 10)()
    ok = (1, 2, 4, 4, 2, 32, 1, 1)   # batch, T, H, W, heads, d, dtype, block_frames

    def call(form, batch, T, H, W, heads, d, dtype, F, buf=out, n=10):
        return lib.gla_plan_describe(form, batch, T, H, W, heads, d, dtype, F, buf, n)

    assert call(0, *ok) == 0
    assert call(3, *ok) == -2 and call(-1, *ok) == -2         # unknown form
    assert call(0, 1, 0, 4, 4, 2, 32, 1, 1) == -2             # empty grid
    assert call(0, 1, 2, 4, 4, 0, 32, 1, 1) == -2             # no heads
    assert call(0, 0, 2, 4, 4, 2, 32, 1, 1) == -2             # no batch
    assert call(1, 1, 2, 4, 4, 2, 32, 1, 0) == -2             # block of no frames
    assert call(0, 1, 2, 4, 4, 2, 48, 1, 1) == -7             # head dim
    assert call(0, 1, 2, 4, 4, 2, 32, 4, 1) == -3             # dtype
    assert call(0, *ok, buf=None, n=10) == -1
    assert call(0, *ok, buf=None, n=0) == 0
    short = (ctypes.c_int * 3)(-1, -1, -1)
    assert call(0, *ok, buf=short, n=2) == 0 and short[2] == -1
    assert list(short[:2]) == [32, 1]
