"""Plain fp64 definition of the backward pass of the windowed softmax branch.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import this module.

The forward is the windowed softmax of the VDN-H3 article ("VDN-Minimax-H3",
icman.com.cn news 81972), sections "Why video models are stuck on attention"
and "What the far field outside the window is": query token n of frame t
attends to every token of frames lo_t..hi_t,

    s_nm = q_n . k_m / sqrt(d),   p_nm = exp(s_nm) / sum_j exp(s_nj),
    o_n  = sum_m p_nm v_m.

The article trains the hybrid attention (section "Training"), which needs the
gradient of this map. Given the upstream gradient g_n = dL/do_n, the chain rule
through the row softmax (dp_nm/ds_nj = p_nm (delta_mj - p_nj)) gives

    dv_m  = sum_n p_nm g_n
    dp_nm = g_n . v_m
    ds_nm = p_nm (dp_nm - sum_j p_nj dp_nj)
    dq_n  = sum_m ds_nm k_m / sqrt(d)
    dk_m  = sum_n ds_nm q_n / sqrt(d)

with every sum over n running over the queries whose window holds key m, and
every sum over m over the keys of query n's window. lse_n = log sum_m
exp(s_nm) is the natural-log normaliser a forward pass can hand to the
backward.

Pinned by (tests/test_oracle_softmax_grad.py): central finite differences of
the forward oracle on tiny inputs, torch autograd of dense fp64 attention when
the window covers every frame and of block-diagonal masked attention at
radius 0, the shift invariance sum_m dk_m = 0, sum_m dv_m = sum_n g_n, a
constant v giving dq = dk = 0, and scipy's logsumexp for lse.

Everything is numpy float64; inputs of lower precision are upcast exactly.
"""

from __future__ import annotations

import math

import numpy as np

_F64 = np.float64


def _window_keys(t: int, S: int, lo, hi):
    return int(lo[t]) * S, (int(hi[t]) + 1) * S


def softmax_lse(q, k, S: int, lo, hi, row_block: int = 512):
    """lse_n = log sum_m exp(q_n . k_m / sqrt(d)) over query n's window, [N]."""
    q = np.asarray(q, _F64)
    k = np.asarray(k, _F64)
    N, d = q.shape
    lse = np.empty(N, dtype=_F64)
    for t in range(N // S):
        k0, k1 = _window_keys(t, S, lo, hi)
        for r0 in range(t * S, (t + 1) * S, row_block):
            r1 = min((t + 1) * S, r0 + row_block)
            s = q[r0:r1] @ k[k0:k1].T / math.sqrt(d)
            m = s.max(axis=1)
            lse[r0:r1] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return lse


def softmax_lse_rows(q, k, S: int, lo, hi, rows):
    """lse_n of :func:`softmax_lse` for the selected query ``rows`` only, one
    row at a time (sampled checks at full size)."""
    q = np.asarray(q)
    d = q.shape[1]
    out = np.empty(len(rows), dtype=_F64)
    for i, n in enumerate(np.asarray(rows, dtype=np.int64)):
        k0, k1 = _window_keys(int(n) // S, S, lo, hi)
        s = np.asarray(k[k0:k1], _F64) @ np.asarray(q[n], _F64) / math.sqrt(d)
        m = s.max()
        out[i] = m + np.log(np.exp(s - m).sum())
    return out


def _block_grad(qs, ks, vs, gs):
    """Gradients of one block of query rows against their common window."""
    d = qs.shape[1]
    s = qs @ ks.T / math.sqrt(d)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    dp = gs @ vs.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = ds @ ks / math.sqrt(d)
    dk = ds.T @ qs / math.sqrt(d)
    dv = p.T @ gs
    return dq, dk, dv


def softmax_branch_grad(q, k, v, g, S: int, lo, hi, row_block: int = 512):
    """(dq, dk, dv) of L = sum_n g_n . o_n for one (batch, head) slice.

    q, k, v, g: [N, d]. Query rows are taken ``row_block`` at a time only to
    bound memory; the key-side sums accumulate over every query frame whose
    window holds the key.
    """
    q = np.asarray(q, _F64)
    k = np.asarray(k, _F64)
    v = np.asarray(v, _F64)
    g = np.asarray(g, _F64)
    N, d = q.shape
    dq = np.zeros((N, d), dtype=_F64)
    dk = np.zeros((N, d), dtype=_F64)
    dv = np.zeros((N, v.shape[1]), dtype=_F64)
    for t in range(N // S):
        k0, k1 = _window_keys(t, S, lo, hi)
        for r0 in range(t * S, (t + 1) * S, row_block):
            r1 = min((t + 1) * S, r0 + row_block)
            bq, bk, bv = _block_grad(q[r0:r1], k[k0:k1], v[k0:k1], g[r0:r1])
            dq[r0:r1] = bq
            dk[k0:k1] += bk
            dv[k0:k1] += bv
    return dq, dk, dv


def softmax_grad_rows(q, k, v, g, S: int, lo, hi, q_rows, k_rows, row_block: int = 1024):
    """dq of the query rows ``q_rows`` and (dk, dv) of the key rows ``k_rows``.

    Same definition as :func:`softmax_branch_grad`, evaluated only where asked
    (sampled checks at sizes where the whole gradient is too slow on a CPU):
    a key row needs every query whose window holds it, and each of those
    queries its own whole window.
    """
    q = np.asarray(q, _F64)
    k = np.asarray(k, _F64)
    v = np.asarray(v, _F64)
    g = np.asarray(g, _F64)
    N, d = q.shape
    sc = 1.0 / math.sqrt(d)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    dq = np.empty((len(q_rows), d), dtype=_F64)
    for i, n in enumerate(q_rows):
        t = int(n) // S
        k0, k1 = _window_keys(t, S, lo, hi)
        bq, _, _ = _block_grad(q[n:n + 1], k[k0:k1], v[k0:k1], g[n:n + 1])
        dq[i] = bq[0]
    dk = np.zeros((len(k_rows), d), dtype=_F64)
    dv = np.zeros((len(k_rows), v.shape[1]), dtype=_F64)
    # group the key rows by the query frames that see them: query frame t
    # sees key m when lo_t <= m // S <= hi_t
    F = N // S
    for t in range(F):
        sel = np.nonzero((k_rows // S >= lo[t]) & (k_rows // S <= hi[t]))[0]
        if len(sel) == 0:
            continue
        k0, k1 = _window_keys(t, S, lo, hi)
        km = k[k_rows[sel]]
        vm = v[k_rows[sel]]
        for r0 in range(t * S, (t + 1) * S, row_block):
            r1 = min((t + 1) * S, r0 + row_block)
            qs, gs = q[r0:r1], g[r0:r1]
            s = qs @ k[k0:k1].T * sc
            mx = s.max(axis=1, keepdims=True)
            e = np.exp(s - mx)
            z = e.sum(axis=1, keepdims=True)
            o = (e / z) @ v[k0:k1]
            delta = (gs * o).sum(axis=1, keepdims=True)  # sum_j p_nj dp_nj
            p = np.exp(qs @ km.T * sc - mx) / z
            ds = p * (gs @ vm.T - delta)
            dk[sel] += ds.T @ qs * sc
            dv[sel] += p.T @ gs
    return dq, dk, dv
