"""Plain fp64 definition of block-sparse routing inside the window.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The H3 acceleration report ("MiniMax H3 加速方案研究报告", section 9.7.3,
path B "Sol-Attn Ampere", and 9.8) describes block-sparse routing for the H3
attention: tokens grouped in 128-token blocks, block means of Q and K, trial
scores q_mean . k_mean^T, and a "mean + tau * std" threshold, with exact
attention only on the blocks that pass. It gives no formula beyond that. The
reading used here, applied to the windowed softmax branch of the hybrid
attention:

* query tiles: the queries of a chunk in tiles of 256 from the chunk's first
  query (the last one partial); key blocks: the 128-token blocks of the global
  token index (block j = tokens 128 j .. 128 j + 127), each cut to the chunk's
  key window [lo * S, (hi + 1) * S);
* q_mean of a tile and k_mean of a block are the plain means over their
  (in-window) tokens; s_j = q_mean . k_mean_j / sqrt(d);
* over the window's key blocks of one query tile, mu = mean_j s_j and sigma =
  the population standard deviation; block j is kept when s_j >= mu + tau *
  sigma, and the block with the largest s_j is always kept;
* every query of the tile attends, with the windowed softmax of the hybrid
  attention, to the keys of its kept blocks only.
tau = -inf keeps every block: the routed branch is then the windowed softmax.
"""

from __future__ import annotations

import math

import numpy as np

from .hybrid_attn import window_bounds

_F64 = np.float64
QTILE = 256
KBLOCK = 128


def route_scores(q, k, S: int, chunk: int, radius: int):
    """Trial scores of every (query tile, key block) of one (batch, head)
    slice: a list over query tiles of (q0, q1, blocks [(k0, k1), ...],
    scores [nb]), in fp64."""
    q = np.asarray(q, _F64)
    k = np.asarray(k, _F64)
    N, d = q.shape
    F = N // S
    lo, hi = window_bounds(F, chunk, radius)
    out = []
    for c0 in range(0, F, chunk):
        qb, qe = c0 * S, min(F, c0 + chunk) * S
        kb, ke = int(lo[c0]) * S, (int(hi[c0]) + 1) * S
        blocks = [(max(kb, j * KBLOCK), min(ke, (j + 1) * KBLOCK))
                  for j in range(kb // KBLOCK, (ke - 1) // KBLOCK + 1)]
        kmean = np.stack([k[a:b].mean(axis=0) for a, b in blocks])
        for q0 in range(qb, qe, QTILE):
            q1 = min(qe, q0 + QTILE)
            s = kmean @ q[q0:q1].mean(axis=0) / math.sqrt(d)
            out.append((q0, q1, blocks, s))
    return out


def route_keep(s, tau: float):
    """Kept blocks of one query tile: s_j >= mean + tau * std, and the
    argmax. Returns a boolean array."""
    s = np.asarray(s, _F64)
    keep = s >= s.mean() + tau * s.std() if np.isfinite(tau) else np.ones(len(s), dtype=bool)
    keep[int(np.argmax(s))] = True
    return keep


def routed_softmax(q, k, v, S: int, chunk: int, radius: int, tau: float, keep=None):
    """Routed windowed softmax output of one slice [N, d] and the kept-block
    masks (a list of boolean arrays, one per query tile in route_scores'
    order). ``keep``: optional masks to use instead of the slice's own
    decisions (the tests pass the GPU's, after checking them)."""
    q = np.asarray(q, _F64)
    k = np.asarray(k, _F64)
    v = np.asarray(v, _F64)
    N, d = q.shape
    o = np.empty((N, v.shape[1]), dtype=_F64)
    masks = []
    for t, (q0, q1, blocks, s) in enumerate(route_scores(q, k, S, chunk, radius)):
        kp = route_keep(s, tau) if keep is None else np.asarray(keep[t], dtype=bool)
        masks.append(kp)
        idx = np.concatenate([np.arange(a, b) for (a, b), kk in zip(blocks, kp) if kk])
        sc = q[q0:q1] @ k[idx].T / math.sqrt(d)
        sc -= sc.max(axis=1, keepdims=True)
        p = np.exp(sc)
        p /= p.sum(axis=1, keepdims=True)
        o[q0:q1] = p @ v[idx]
    return o, masks
