"""Pins of the block oracle (oracle/block.py): the stated 3D RoPE and the
block around the hybrid attention (CPU only)."""

import math

import numpy as np

import oracle

RNG = np.random.default_rng(77)


def test_rope_pairs_split():
    assert oracle.rope_pairs(128) == (22, 21, 21)
    assert oracle.rope_pairs(64) == (12, 10, 10)
    assert oracle.rope_pairs(8) == (2, 1, 1)


def test_rope_hand_worked_d8():
    # d = 8: pairs 0, 1 on time (P = 2), pair 2 on rows, pair 3 on columns.
    # Token of frame 1, row 2, column 3 (S = 20 tokens per frame, 5 columns):
    # n = 1 * 20 + 2 * 5 + 3 = 33; angles 1, 1 * 100^-1 = 0.01, 2, 3.
    S, gw = 20, 5
    x = np.zeros((40, 8))
    x[33] = [1.0, 2.0, -0.5, 0.25, 3.0, -1.0, 0.5, 0.75]
    got = oracle.rope3d(x, S, gw, theta=10000.0)[33]
    want = []
    for (a, b), ang in zip(((1.0, 2.0), (-0.5, 0.25), (3.0, -1.0), (0.5, 0.75)),
                           (1.0, 0.01, 2.0, 3.0)):
        want += [a * math.cos(ang) - b * math.sin(ang), a * math.sin(ang) + b * math.cos(ang)]
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_rope_invariants():
    S, gw, d = 12, 4, 16
    N = 5 * S
    x = RNG.standard_normal((N, d))
    r = oracle.rope3d(x, S, gw)
    # a rotation: every channel pair keeps its length
    assert np.allclose(np.hypot(r[:, 0::2], r[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]),
                       rtol=1e-14)
    # token 0 (frame 0, row 0, column 0) is not turned
    assert np.allclose(r[0], x[0], rtol=0, atol=0)
    # relative positions: the score of two tokens depends on their offsets
    # only: moving both by one frame, or both by one column, keeps q.k
    q, k = RNG.standard_normal(d), RNG.standard_normal(d)
    X = np.zeros((N, d))

    def score(n1, n2):
        X[:] = 0
        X[n1] = q
        Rq = oracle.rope3d(X, S, gw)[n1]
        X[:] = 0
        X[n2] = k
        Rk = oracle.rope3d(X, S, gw)[n2]
        return float(Rq @ Rk)

    base = score(1 * S + 5, 2 * S + 2)           # frame 1 (1, 1) vs frame 2 (0, 2)
    assert abs(score(2 * S + 5, 3 * S + 2) - base) < 1e-12   # both one frame later
    assert abs(score(1 * S + 6, 2 * S + 3) - base) < 1e-12   # both one column right
    assert abs(score(1 * S + 9, 2 * S + 6) - base) < 1e-12   # both one row down
    assert abs(score(1 * S + 5, 2 * S + 3) - base) > 1e-6    # a different offset


def _block_case(H=2, d=16, F=6, S=8, gw=4):
    D = H * d
    N = F * S
    x = RNG.standard_normal((N, D))
    wq = RNG.standard_normal((3 * D, D)) / math.sqrt(D)
    wo = RNG.standard_normal((D, D)) / math.sqrt(D)
    beta = RNG.uniform(0, 1, (H, N))
    alpha = RNG.uniform(0.8, 1, (H, F, d))
    gate = RNG.standard_normal((H, N, d))
    st = RNG.standard_normal((H, d, d)) / math.sqrt(d)
    ck = RNG.standard_normal((H, d, 4)) * 0.5
    cv = RNG.standard_normal((H, d, 4)) * 0.5
    return dict(x=x, w_qkv=wq, w_o=wo, beta=beta, alpha=alpha, gate=gate, text_states=st,
                conv_k=ck, conv_v=cv, w=np.ones(d), H=H, S=S, grid_w=gw, chunk=2, radius=1)


def test_block_head_permutation_and_linearity():
    c = _block_case()
    y = oracle.block_fwd(**c)
    # swapping the two heads everywhere (their rows of W_qkv in q, k and v,
    # their per-head inputs, their columns of W_o) leaves y unchanged
    H, d = c["H"], c["w"].shape[0]
    D = H * d
    perm = np.concatenate([np.arange(d, 2 * d), np.arange(0, d)])
    rows = np.concatenate([perm, D + perm, 2 * D + perm])
    c2 = dict(c, w_qkv=c["w_qkv"][rows], w_o=c["w_o"][:, perm], beta=c["beta"][::-1],
              alpha=c["alpha"][::-1], gate=c["gate"][::-1], text_states=c["text_states"][::-1],
              conv_k=c["conv_k"][::-1], conv_v=c["conv_v"][::-1])
    assert np.allclose(oracle.block_fwd(**c2), y, rtol=1e-12, atol=1e-13)
    # the output projection is linear
    assert np.allclose(oracle.block_fwd(**dict(c, w_o=2.0 * c["w_o"])), 2.0 * y, rtol=1e-13,
                       atol=1e-14)
    # a zero W_o gives zero
    assert not np.any(oracle.block_fwd(**dict(c, w_o=np.zeros_like(c["w_o"]))))


def test_block_selection_weights_reduce_to_the_attention():
    # W_qkv selecting x's own head channels for q, k and v and W_o = I: y's
    # head h columns are the hybrid attention of x_h with q = k = v = x_h and
    # the softmax branch on RoPE3D(x_h)
    c = _block_case()
    H, d = c["H"], c["w"].shape[0]
    D = H * d
    c["w_qkv"] = np.concatenate([np.eye(D)] * 3)
    c["w_o"] = np.eye(D)
    y = oracle.block_fwd(**c)
    for h in range(H):
        xh = c["x"][:, h * d:(h + 1) * d]
        r = oracle.rope3d(xh, c["S"], c["grid_w"])
        ref = oracle.hybrid_attn_head(xh, xh, xh, c["beta"][h], c["alpha"][h], c["gate"][h],
                                      c["text_states"][h], c["conv_k"][h], c["conv_v"][h],
                                      c["w"], c["S"], c["chunk"], c["radius"], q_rope=r,
                                      k_rope=r)[0]
        assert np.allclose(y[:, h * d:(h + 1) * d], ref, rtol=1e-12, atol=1e-14)
