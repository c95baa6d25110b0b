"""Pins of the block-sparse routing oracle (oracle/routing.py, CPU only)."""

import math

import numpy as np

import oracle

RNG = np.random.default_rng(91)


def _case(F=12, S=100, d=16, drift=True):
    q, k, v = (RNG.standard_normal((F * S, d)) for _ in range(3))
    if drift:  # give blocks distinct means, as video tokens of a scene have
        nb = -(-F * S // 50)
        k += np.repeat(RNG.standard_normal((nb, d)), 50, axis=0)[:F * S]
        q += 0.5 * np.repeat(RNG.standard_normal((nb, d)), 50, axis=0)[:F * S]
    return q, k, v


def test_keep_everything_is_the_windowed_softmax():
    q, k, v = _case()
    lo, hi = oracle.window_bounds(12, 5, 1)
    o, masks = oracle.routed_softmax(q, k, v, 100, 5, 1, -math.inf)
    assert all(m.all() for m in masks)
    assert np.allclose(o, oracle.softmax_branch(q, k, v, 100, lo, hi), rtol=1e-12, atol=1e-14)


def test_scores_and_decisions_brute_force():
    F, S, d, chunk, radius, tau = 7, 90, 8, 3, 1, 0.8
    q, k, v = _case(F, S, d)
    got = oracle.route_scores(q, k, S, chunk, radius)
    tiles = []
    for c0 in range(0, F, chunk):
        lo_f = max(0, c0 - radius * chunk)
        hi_f = min(F - 1, c0 + (radius + 1) * chunk - 1)
        kb, ke = lo_f * S, (hi_f + 1) * S
        qb, qe = c0 * S, min(F, c0 + chunk) * S
        for q0 in range(qb, qe, 256):
            tiles.append((q0, min(qe, q0 + 256), kb, ke))
    assert len(tiles) == len(got)
    for (q0, q1, kb, ke), (g0, g1, blocks, s) in zip(tiles, got):
        assert (q0, q1) == (g0, g1)
        qm = [sum(q[n, c] for n in range(q0, q1)) / (q1 - q0) for c in range(d)]
        ref_blocks, ref_s = [], []
        j = kb // 128
        while j * 128 < ke:
            a, b = max(kb, j * 128), min(ke, (j + 1) * 128)
            km = [sum(k[n, c] for n in range(a, b)) / (b - a) for c in range(d)]
            ref_blocks.append((a, b))
            ref_s.append(sum(x * y for x, y in zip(qm, km)) / math.sqrt(d))
            j += 1
        assert blocks == ref_blocks
        assert np.allclose(s, ref_s, rtol=1e-12, atol=1e-14)
        mu = sum(ref_s) / len(ref_s)
        sd = math.sqrt(sum((x - mu) ** 2 for x in ref_s) / len(ref_s))
        keep = oracle.route_keep(s, tau)
        best = max(range(len(ref_s)), key=lambda i: ref_s[i])
        for i, x in enumerate(ref_s):
            assert keep[i] == (x >= mu + tau * sd or i == best)


def test_density_falls_with_tau_and_never_empty():
    q, k, v = _case()
    prev = None
    for tau in (-1.0, 0.0, 0.5, 1.0, 2.0, 10.0):
        _, masks = oracle.routed_softmax(q, k, v, 100, 5, 1, tau)
        assert all(m.sum() >= 1 for m in masks)
        kept = sum(int(m.sum()) for m in masks)
        assert prev is None or kept <= prev
        prev = kept
    assert prev == len(masks)  # tau = 10: only each tile's best block


def test_given_masks_restrict_the_keys():
    # with masks given, a tile's output is the softmax over its kept keys
    F, S, d = 10, 60, 8
    q, k, v = _case(F, S, d, drift=False)
    tiles = oracle.route_scores(q, k, S, 5, 1)
    masks = [np.zeros(len(t[2]), dtype=bool) for t in tiles]
    for m in masks:
        m[::2] = True
    o, _ = oracle.routed_softmax(q, k, v, S, 5, 1, 0.0, keep=masks)
    q0, q1, blocks, _ = tiles[1]
    idx = np.concatenate([np.arange(a, b) for (a, b), kk in zip(blocks, masks[1]) if kk])
    n = q0 + 3
    s = k[idx] @ q[n] / math.sqrt(d)
    p = np.exp(s - s.max())
    assert np.allclose(o[n], (p / p.sum()) @ v[idx], rtol=1e-12, atol=1e-14)
