"""Plain fp64 definition of the attention block around the hybrid attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The VDN-H3 article ("VDN-Minimax-H3", icman.com.cn news 81972) says, in "Why
video models are stuck on attention", that one QKV projection feeds both
branches and that their outputs are summed, and in "Step 1: NoPE features"
that the softmax branch uses RoPE'd q and k while the linear branch takes
them without position encoding. It does not define the projections' shapes or
the RoPE. The block here states them:

* shared QKV projection of the block input x [N, D] (D = H * d):
  [q | k | v] = x W_qkv^T with W_qkv [3 H d, D] (rows = output features,
  q first, then k, then v; head h of each takes features h d .. h d + d - 1);
* 3D RoPE on the softmax branch's q and k, over the token's (frame, row,
  column) on the latent grid (S tokens per frame in raster order, grid_w
  columns): the d / 2 channel pairs (2i, 2i + 1) split into p_t =
  d/2 - 2 floor(d/6) time pairs, then p_h = floor(d/6) row pairs, then
  p_w = floor(d/6) column pairs; pair u of an axis with P pairs turns by
  angle pos * theta^(-u / P) (pos = the token's frame, row or column index);
* the hybrid attention of the slice (oracle.hybrid_attn_head), with the raw
  q, k for the linear branch and the rotated ones for the softmax branch;
* output projection y = concat_h(out_h) W_o^T with W_o [D, D].
"""

from __future__ import annotations

import numpy as np

from .hybrid_attn import hybrid_attn_head

_F64 = np.float64


def rope_pairs(d: int):
    """(p_t, p_h, p_w): channel pairs per axis."""
    ph = (d // 2) // 3
    return d // 2 - 2 * ph, ph, ph


def rope_angles(N: int, S: int, grid_w: int, d: int, theta: float = 10000.0):
    """Angle of every (token, channel pair), [N, d / 2] in fp64."""
    pt, ph, pw = rope_pairs(d)
    n = np.arange(N)
    s = n % S
    pos = (n // S, s // grid_w, s % grid_w)
    ang = np.empty((N, d // 2), dtype=_F64)
    i0 = 0
    for p, P in zip(pos, (pt, ph, pw)):
        u = np.arange(P, dtype=_F64)
        ang[:, i0:i0 + P] = np.asarray(p, _F64)[:, None] * theta ** (-u / P)[None, :]
        i0 += P
    return ang


def rope3d(x, S: int, grid_w: int, theta: float = 10000.0):
    """Rotate each channel pair (2i, 2i+1) of x [N, d] by its angle:
    (a, b) -> (a cos - b sin, a sin + b cos)."""
    x = np.asarray(x, _F64)
    N, d = x.shape
    ang = rope_angles(N, S, grid_w, d, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = a * c - b * s
    out[:, 1::2] = a * s + b * c
    return out


def block_fwd(x, w_qkv, w_o, beta, alpha, gate, text_states, conv_k, conv_v, w,
              H: int, S: int, grid_w: int, theta: float = 10000.0, chunk: int = 5,
              radius: int = 1, rule: str = "vdn_solve", c: float = 0.5,
              text_scale: float = 0.5, eps: float = 1e-6, round_to=None):
    """Block output y [N, D] for one batch element.

    x [N, D]; w_qkv [3 D, D]; w_o [D, D]; beta [H, N]; alpha [H, F, d];
    gate [H, N, d]; text_states [H, d, d] or None; conv_k, conv_v [H, d, 4];
    w [d]. ``round_to``: optional function applied to q, k, v, their rotations
    and the attention output before they are used (the rounding points of an
    implementation that stores them in a narrower type); None = fp64
    throughout.
    """
    x = np.asarray(x, _F64)
    N, D = x.shape
    d = D // H
    rnd = (lambda a: a) if round_to is None else round_to
    qkv = x @ np.asarray(w_qkv, _F64).T
    outs = []
    for h in range(H):
        q = rnd(qkv[:, h * d:(h + 1) * d])
        k = rnd(qkv[:, D + h * d:D + (h + 1) * d])
        v = rnd(qkv[:, 2 * D + h * d:2 * D + (h + 1) * d])
        qr = rnd(rope3d(qkv[:, h * d:(h + 1) * d], S, grid_w, theta))
        kr = rnd(rope3d(qkv[:, D + h * d:D + (h + 1) * d], S, grid_w, theta))
        st = None if text_states is None else text_states[h]
        o = hybrid_attn_head(q, k, v, beta[h], alpha[h], gate[h], st, conv_k[h], conv_v[h], w,
                             S, chunk, radius, rule, c, text_scale, eps, q_rope=qr,
                             k_rope=kr)[0]
        outs.append(rnd(o))
    return np.concatenate(outs, axis=1) @ np.asarray(w_o, _F64).T
