"""Pins of the oracle's windowed-softmax backward (CPU only).

The gradient is the chain rule through the windowed softmax of the VDN-H3
article ("What the far field outside the window is"); these tests tie it to
things other than its own formula: finite differences of the forward oracle,
torch autograd of dense attention where the window reduces to it, and the
invariances of softmax attention.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def _draw(rng, N, d, scale=1.0):
    return rng.standard_normal((N, d)) * scale


def _loss(q, k, v, g, S, lo, hi):
    return float((oracle.softmax_branch(q, k, v, S, lo, hi) * g).sum())


@pytest.mark.parametrize("F,S,d,chunk,radius", [
    (4, 3, 4, 2, 0),   # block-diagonal chunks
    (5, 2, 4, 2, 1),   # overlapping windows, partial last chunk
    (6, 2, 3, 1, 1),   # chunk of one frame
])
def test_grad_matches_central_differences(F, S, d, chunk, radius):
    rng = np.random.default_rng([41, F, S, d])
    N = F * S
    q, k, v, g = (_draw(rng, N, d) for _ in range(4))
    lo, hi = oracle.window_bounds(F, chunk, radius)
    dq, dk, dv = oracle.softmax_branch_grad(q, k, v, g, S, lo, hi)
    h = 1e-5
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            up = _loss(q, k, v, g, S, lo, hi)
            x[idx] = old - h
            dn = _loss(q, k, v, g, S, lo, hi)
            x[idx] = old
            num[idx] = (up - dn) / (2 * h)
        np.testing.assert_allclose(dx, num, rtol=1e-6, atol=1e-8)


def _torch_grad(q, k, v, g, mask):
    """Dense fp64 attention through torch autograd, keys masked per query."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = tq @ tk.T / math.sqrt(q.shape[1])
    s = s.masked_fill(~torch.tensor(mask), float("-inf"))
    o = torch.softmax(s, dim=1) @ tv
    (o * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("radius", [0, 3])
def test_grad_matches_torch_autograd(radius):
    # radius 3 covers every chunk of 7 frames (textbook full attention);
    # radius 0 is attention within each chunk (block-diagonal mask)
    F, S, d, chunk = 7, 5, 8, 2
    rng = np.random.default_rng([42, radius])
    N = F * S
    q, k, v, g = (_draw(rng, N, d) for _ in range(4))
    lo, hi = oracle.window_bounds(F, chunk, radius)
    frame = np.arange(N) // S
    if radius == 3:
        mask = np.ones((N, N), dtype=bool)
    else:
        mask = (frame[:, None] // chunk) == (frame[None, :] // chunk)
    ref = _torch_grad(q, k, v, g, mask)
    got = oracle.softmax_branch_grad(q, k, v, g, S, lo, hi, row_block=3)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_grad_invariances():
    # adding one vector to every key shifts each query's scores by a constant
    # (its window gets the shift on every key): the output does not move, so
    # the key gradients sum to zero; the rows of p sum to one, so the value
    # gradients sum to the upstream gradients
    F, S, d = 13, 7, 16
    rng = np.random.default_rng(43)
    q, k, v, g = (_draw(rng, F * S, d) for _ in range(4))
    for chunk, radius in ((5, 1), (3, 0), (2, 2)):
        lo, hi = oracle.window_bounds(F, chunk, radius)
        dq, dk, dv = oracle.softmax_branch_grad(q, k, v, g, S, lo, hi)
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=0), g.sum(axis=0), rtol=1e-12, atol=1e-12)
        assert np.abs(dq).max() > 0.01 and np.abs(dk).max() > 0.01


def test_grad_constant_values():
    # every value row equal: the output is that row whatever q and k are
    F, S, d = 9, 4, 8
    rng = np.random.default_rng(44)
    q, k, g = (_draw(rng, F * S, d) for _ in range(3))
    v = np.tile(rng.standard_normal(d), (F * S, 1))
    lo, hi = oracle.window_bounds(F, 3, 1)
    dq, dk, dv = oracle.softmax_branch_grad(q, k, v, g, S, lo, hi)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    assert np.abs(dv).max() > 0.1


def test_lse_matches_logsumexp_and_output():
    F, S, d = 8, 6, 16
    rng = np.random.default_rng(45)
    q, k, v = (_draw(rng, F * S, d, 3.0) for _ in range(3))
    lo, hi = oracle.window_bounds(F, 3, 1)
    lse = oracle.softmax_lse(q, k, S, lo, hi, row_block=4)
    o = oracle.softmax_branch(q, k, v, S, lo, hi)
    rows = np.array([0, 7, 23, 47])
    lse_rows = oracle.softmax_lse_rows(q, k, S, lo, hi, rows)
    for n in range(F * S):
        t = n // S
        k0, k1 = lo[t] * S, (hi[t] + 1) * S
        s = q[n] @ k[k0:k1].T / math.sqrt(d)
        assert lse[n] == pytest.approx(scipy.special.logsumexp(s), rel=1e-14)
        if n in rows:
            i = int(np.nonzero(rows == n)[0][0])
            assert lse_rows[i] == pytest.approx(scipy.special.logsumexp(s), rel=1e-14)
        np.testing.assert_allclose(np.exp(s - lse[n]) @ v[k0:k1], o[n], rtol=1e-12, atol=1e-14)


def test_grad_rows_agree_with_whole_gradient():
    F, S, d = 11, 9, 8
    rng = np.random.default_rng(46)
    q, k, v, g = (_draw(rng, F * S, d) for _ in range(4))
    lo, hi = oracle.window_bounds(F, 3, 1)
    dq, dk, dv = oracle.softmax_branch_grad(q, k, v, g, S, lo, hi)
    qr = np.array([0, 5, 40, 98])
    kr = np.array([1, 27, 28, 60, 97])
    rq, rk, rv = oracle.softmax_grad_rows(q, k, v, g, S, lo, hi, qr, kr, row_block=4)
    np.testing.assert_allclose(rq, dq[qr], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rk, dk[kr], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rv, dv[kr], rtol=1e-12, atol=1e-14)
