"""Oracle: plain, slow, fp64 CPU evaluation of gated bidirectional ReLU linear attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP kernels.

What it computes (per head, tokens n, j of one video-latent grid):

* q and k are RMS-normalised over the head dimension before the feature map
  (SANA-Video 2.0 digest, prelims "gated bilinear linear attention": RoPE acts
  on the normalised query/key).  No learnable weight; the call's eps.
* phi = ReLU (same passage; SANA-Video notes, key design 1).
* 3D RoPE is applied AFTER phi, i.e. RoPE(phi(x)), and only in the numerator;
  the denominator uses the un-rotated phi so it stays positive (SANA-Video
  notes, key design 1, "RoPE(ReLU(x))" and the numerator-only placement).
* State  S = sum_n beta_n v_n (R_n phi(k_n))^T   (d_v x d_k), key sum
  z = sum_n phi(k_n)  (digest, prelims "linear attention": the state is a sum of
  v_n (beta_n k_n)^T; reader, appendix F.7: "gated RoPE-rotated linear state";
  notes, key design 2: key sum of phi(K)).
* o_j = w * RMSNorm[ sigmoid(g_j) * (S R_j phi(q_j)) / (phi(q_j) . z + eps) ]
  (digest, prelims "gated bilinear linear attention", output formula; W_o is
  not part of the operator here).  Bidirectional: every j sees every n.
* Block-causal mode: the running sums of S and z are carried across blocks of
  latent frames (notes, key design 2: cumulative state + key sum form a
  constant-memory cache).  Tokens of block b see blocks <= b; inside a block
  attention is bidirectional.
* Token-causal mode: token i sees the tokens before it in row-major order
  (notes, key design 2: the causal form as running sums up to i - 1), or
  also itself; both readings are evaluated.

Readings where the pages are silent (each listed with its reason in the
design notes of the repository):
* RoPE split of the head dim into (d/4, 3d/8, 3d/8) channels for (t, h, w),
  contiguous in that order; within an axis slice, pair i is channels
  (2i, 2i+1) and rotates by pos * base^(-2i/d_axis), base 10000, positions
  counted from 0; rotation (u, w) -> (u cos a - w sin a, u sin a + w cos a).
* Token order n = (t*H + y)*W + x; tensors are [N, heads, d]; beta is
  [N, heads]; the output RMSNorm weight w is [d], shared by heads; one eps is
  used for the q/k normalisation, the denominator and the output RMSNorm.
* z carries neither beta nor RoPE.

Everything is evaluated in float64 from the exact input values.
"""
from __future__ import annotations

import numpy as np

ROPE_BASE = 10000.0

__all__ = [
    "ROPE_BASE",
    "rms_normalize",
    "relu",
    "sigmoid",
    "rope_axis_widths",
    "rope_angles",
    "rope_rotate",
    "head_features",
    "gla_forward",
    "gla_block_causal_forward",
    "gla_token_causal_forward",
    "gla_token_causal_rows",
    "block_bounds",
]


def rms_normalize(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis (no weight)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def relu(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0)


def sigmoid(x: np.ndarray) -> np.ndarray:
    # for x below about -709, exp(-x) overflows to inf and the value is 0, the
    # function's limit; the overflow is expected and not reported
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def rope_axis_widths(d: int) -> tuple:
    """Channels given to the (t, h, w) axes: (d/4, 3d/8, 3d/8)."""
    if d % 16 != 0:
        raise ValueError("head dim must be a multiple of 16 for the 3D RoPE split")
    return (d // 4, 3 * d // 8, 3 * d // 8)


def rope_angles(T: int, H: int, W: int, d: int, base: float = ROPE_BASE,
                pos_offset=(0, 0, 0)) -> np.ndarray:
    """Rotation angle of every (token, channel pair): float64 [N, d/2].

    Pair p covers channels (2p, 2p+1).  The first d/8 pairs follow the frame
    index t, the next 3d/16 the row y, the last 3d/16 the column x.  Pair i of
    an axis of width d_a turns by pos * base^(-2i/d_a).
    """
    widths = rope_axis_widths(d)
    t = np.arange(T, dtype=np.float64) + pos_offset[0]
    y = np.arange(H, dtype=np.float64) + pos_offset[1]
    x = np.arange(W, dtype=np.float64) + pos_offset[2]
    tt, yy, xx = np.meshgrid(t, y, x, indexing="ij")
    pos = [tt.reshape(-1), yy.reshape(-1), xx.reshape(-1)]
    cols = []
    for a, da in enumerate(widths):
        i = np.arange(da // 2, dtype=np.float64)
        freq = base ** (-2.0 * i / da)
        cols.append(pos[a][:, None] * freq[None, :])
    return np.concatenate(cols, axis=1)


def rope_rotate(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate channel pairs (2p, 2p+1) of x [N, d] by angles [N, d/2]."""
    x = np.asarray(x, dtype=np.float64)
    c = np.cos(angles)
    s = np.sin(angles)
    u = x[..., 0::2]
    w = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = u * c - w * s
    out[..., 1::2] = u * s + w * c
    return out


def head_features(xh: np.ndarray, angles, eps: float):
    """For one head's q or k rows [N, d]: (phi, rotated phi)."""
    p = relu(rms_normalize(xh, eps))
    r = p if angles is None else rope_rotate(p, angles)
    return p, r


def _head(a: np.ndarray, h: int) -> np.ndarray:
    return np.asarray(a[:, h, :], dtype=np.float64)


def _state(beta_h, v_h, pk, rk):
    """S = sum_n beta_n v_n rk_n^T  (d_v x d_k) and z = sum_n phi(k_n)."""
    bv = np.asarray(beta_h, dtype=np.float64)[:, None] * v_h
    return bv.T @ rk, pk.sum(axis=0)


def _output_rows(pq, rq, S, z, gh, w, eps):
    num = rq @ S.T                     # S R phi(q_j)
    den = pq @ z + eps                 # phi(q_j) . z + eps
    x = sigmoid(gh) * num / den[:, None]
    o = w[None, :] * rms_normalize(x, eps)
    return o, num, den, x


def gla_forward(q, k, v, beta, g, rms_w, grid, eps, rope=True, heads=None, rows=None,
                return_parts=False, pos_offset=(0, 0, 0)):
    """Bidirectional operator.

    q, k, v, g: [N, H_heads, d]; beta: [N, H_heads]; rms_w: [d]; grid=(T,H,W).
    heads: optional list of head indices to evaluate (default all).
    rows: optional token indices at which to evaluate the output (the state
    always sums over every token).
    Returns out [len(rows) or N, len(heads), d] float64, or a dict with
    out, S [h,d,d], z [h,d], num, den, x when return_parts.
    """
    T, H, W = grid
    N = T * H * W
    q = np.asarray(q)
    if q.shape[0] != N:
        raise ValueError("token count does not match the grid")
    d = q.shape[2]
    head_ids = list(range(q.shape[1])) if heads is None else list(heads)
    row_ids = np.arange(N) if rows is None else np.asarray(rows)
    ang = rope_angles(T, H, W, d, pos_offset=pos_offset) if rope else None
    ang_rows = None if ang is None else ang[row_ids]
    w = np.asarray(rms_w, dtype=np.float64)
    outs, Ss, zs, nums, dens, xs = [], [], [], [], [], []
    for h in head_ids:
        pk, rk = head_features(_head(k, h), ang, eps)
        S, z = _state(beta[:, h], _head(v, h), pk, rk)
        pq, rq = head_features(np.asarray(q[row_ids, h, :], dtype=np.float64), ang_rows, eps)
        o, num, den, x = _output_rows(pq, rq, S, z, np.asarray(g[row_ids, h, :], dtype=np.float64), w, eps)
        outs.append(o)
        if return_parts:
            Ss.append(S); zs.append(z); nums.append(num); dens.append(den); xs.append(x)
    out = np.stack(outs, axis=1)
    if not return_parts:
        return out
    return {"out": out, "S": np.stack(Ss), "z": np.stack(zs), "num": np.stack(nums, axis=1),
            "den": np.stack(dens, axis=1), "x": np.stack(xs, axis=1)}


def block_bounds(T: int, H: int, W: int, block_frames: int):
    """Token ranges [start, end) of the blocks of block_frames latent frames;
    the last block may be shorter."""
    if block_frames < 1:
        raise ValueError("block_frames must be >= 1")
    hw = H * W
    return [(b * hw, min(b + block_frames, T) * hw) for b in range(0, T, block_frames)]


def gla_block_causal_forward(q, k, v, beta, g, rms_w, grid, eps, block_frames, S0=None, z0=None,
                             rope=True, return_parts=False, pos_offset=(0, 0, 0)):
    """Block-causal operator with a carried (S, z) state.

    Blocks of block_frames frames are visited in order.  The running state starts
    from (S0, z0) (zeros if None); each block first adds its own tokens'
    contributions, then its tokens read the running state (inclusive of their own
    block).  Returns (out [N, heads, d], S_final [heads, d, d], z_final [heads, d]),
    or a dict with the per-block states when return_parts.
    """
    T, H, W = grid
    N = T * H * W
    q = np.asarray(q)
    nh, d = q.shape[1], q.shape[2]
    ang = rope_angles(T, H, W, d, pos_offset=pos_offset) if rope else None
    w = np.asarray(rms_w, dtype=np.float64)
    out = np.zeros((N, nh, d))
    S_fin = np.zeros((nh, d, d))
    z_fin = np.zeros((nh, d))
    bounds = block_bounds(T, H, W, block_frames) if N > 0 else []
    block_states = []
    for h in range(nh):
        S = np.zeros((d, d)) if S0 is None else np.asarray(S0[h], dtype=np.float64).copy()
        z = np.zeros(d) if z0 is None else np.asarray(z0[h], dtype=np.float64).copy()
        pk, rk = head_features(_head(k, h), ang, eps)
        pq, rq = head_features(_head(q, h), ang, eps)
        vh = _head(v, h)
        per_block = []
        for (s, e) in bounds:
            dS, dz = _state(beta[s:e, h], vh[s:e], pk[s:e], rk[s:e])
            S = S + dS
            z = z + dz
            o, _, _, _ = _output_rows(pq[s:e], rq[s:e], S, z, _head(g, h)[s:e], w, eps)
            out[s:e, h, :] = o
            per_block.append((S.copy(), z.copy()))
        S_fin[h] = S
        z_fin[h] = z
        block_states.append(per_block)
    if not return_parts:
        return out, S_fin, z_fin
    return {"out": out, "S": S_fin, "z": z_fin, "block_states": block_states}


def gla_token_causal_forward(q, k, v, beta, g, rms_w, grid, eps, include_self=True, S0=None, z0=None,
                             rope=True, return_parts=False, pos_offset=(0, 0, 0)):
    """Token-level causal operator (SANA-Video notes, key design 2: causal
    linear attention as running sums of the per-token states and key sums).

    Tokens are taken in row-major (t, y, x) order.  Token i reads the carried
    state (S0, z0) plus the tokens j <= i (include_self) or j < i (strictly
    earlier, the notes' sums up to i - 1).  Written as masked kernel attention
    with M_ij = [j <= i] (or [j < i]):
        num_i = S0 rq_i + sum_j M_ij beta_j (rk_j . rq_i) v_j
        den_i = phi(q_i) . (z0 + sum_j M_ij phi(k_j)) + eps
        out_i = w * rmsnorm(sigmoid(g_i) * num_i / den_i)
    The state after the call is S0 + sum_j beta_j v_j rk_j^T, z0 + sum_j phi(k_j).
    Returns (out [N, heads, d], S_final, z_final), or a dict with num and den
    as well when return_parts.  Dense N x N per head: for test sizes only.
    """
    T, H, W = grid
    N = T * H * W
    q = np.asarray(q)
    nh, d = q.shape[1], q.shape[2]
    ang = rope_angles(T, H, W, d, pos_offset=pos_offset) if rope else None
    w = np.asarray(rms_w, dtype=np.float64)
    mask = np.tril(np.ones((N, N)), 0 if include_self else -1)
    out = np.zeros((N, nh, d))
    nums = np.zeros((N, nh, d))
    dens = np.zeros((N, nh))
    S_fin = np.zeros((nh, d, d))
    z_fin = np.zeros((nh, d))
    for h in range(nh):
        S = np.zeros((d, d)) if S0 is None else np.asarray(S0[h], dtype=np.float64)
        z = np.zeros(d) if z0 is None else np.asarray(z0[h], dtype=np.float64)
        pk, rk = head_features(_head(k, h), ang, eps)
        pq, rq = head_features(_head(q, h), ang, eps)
        bh = np.asarray(beta[:, h], dtype=np.float64)
        vh = _head(v, h)
        num = rq @ S.T + (mask * (rq @ rk.T) * bh[None, :]) @ vh
        den = pq @ z + (mask * (pq @ pk.T)).sum(axis=1) + eps
        x = sigmoid(_head(g, h)) * num / den[:, None]
        out[:, h, :] = w[None, :] * rms_normalize(x, eps)
        nums[:, h, :] = num
        dens[:, h] = den
        dS, dz = _state(bh, vh, pk, rk)
        S_fin[h] = S + dS
        z_fin[h] = z + dz
    if not return_parts:
        return out, S_fin, z_fin
    return {"out": out, "S": S_fin, "z": z_fin, "num": nums, "den": dens}


def gla_token_causal_rows(q, k, v, beta, g, rms_w, grid, eps, rows, heads=None, include_self=True, S0=None,
                          z0=None, pos_offset=(0, 0, 0)):
    """Token-causal output at chosen tokens only, for sequences too long for the
    dense N x N form (SANA-Video notes, key design 2: the causal form as a
    running state and key sum).  The running sums are advanced from one chosen
    token to the next by adding the tokens in between:
        S(i) = S0 + sum_{j <= i} beta_j v_j rk_j^T,  z(i) = z0 + sum_{j <= i} phi(k_j)
    and token i reads S(i), z(i) (include_self) or S(i - 1), z(i - 1).
    Returns out [len(rows), len(heads), d] in the order of `rows`.
    """
    T, H, W = grid
    q = np.asarray(q)
    d = q.shape[2]
    head_ids = list(range(q.shape[1])) if heads is None else list(heads)
    row_ids = np.asarray(rows, dtype=np.int64)
    order = np.argsort(row_ids, kind="stable")
    ang = rope_angles(T, H, W, d, pos_offset=pos_offset)
    w = np.asarray(rms_w, dtype=np.float64)
    out = np.zeros((len(row_ids), len(head_ids), d))
    for hi, h in enumerate(head_ids):
        S = np.zeros((d, d)) if S0 is None else np.asarray(S0[h], dtype=np.float64).copy()
        z = np.zeros(d) if z0 is None else np.asarray(z0[h], dtype=np.float64).copy()
        pk, rk = head_features(_head(k, h), ang, eps)
        vh = _head(v, h)
        done = 0                     # tokens [0, done) are in (S, z)
        for m in order:
            i = int(row_ids[m])
            upto = i + 1 if include_self else i
            if upto > done:
                dS, dz = _state(beta[done:upto, h], vh[done:upto], pk[done:upto], rk[done:upto])
                S = S + dS
                z = z + dz
                done = upto
            pq, rq = head_features(np.asarray(q[i:i + 1, h, :], dtype=np.float64), ang[i:i + 1], eps)
            o, _, _, _ = _output_rows(pq, rq, S, z, np.asarray(g[i:i + 1, h, :], dtype=np.float64), w, eps)
            out[m, hi, :] = o[0]
    return out
