"""Pins of the oracle's linear-branch gradient (CPU only).

The torch float64 transcription of the linear branch must reproduce the numpy
oracle's output, and its autograd gradient must match central finite
differences of the numpy oracle for every input tensor (VDN-H3 article,
"Step 1" .. "Step 5", "Text state").
"""

import numpy as np
import pytest
import torch

import oracle


def _case(seed, F=6, S=3, d=4, text=True):
    rng = np.random.default_rng(seed)
    N = F * S
    return dict(
        q=rng.standard_normal((N, d)), k=rng.standard_normal((N, d)),
        v=rng.standard_normal((N, d)), beta=rng.random(N),
        alpha=0.8 + 0.2 * rng.random((F, d)), gate=rng.standard_normal((N, d)),
        S_text=rng.standard_normal((d, d)) if text else None,
        conv_k=0.5 * rng.standard_normal((d, 4)), conv_v=0.5 * rng.standard_normal((d, 4)),
        w=0.5 + rng.random(d))


@pytest.mark.parametrize("rule", oracle.RULES)
def test_torch_forward_matches_numpy_oracle(rule):
    x = _case(60)
    S = 3
    y_np, _ = oracle.linear_branch(*(x[n] for n in oracle.linear_grad.NAMES), S, 2, 1, rule,
                                   0.5, 0.5, 1e-6)
    ts = [None if x[n] is None else torch.tensor(x[n], dtype=torch.float64)
          for n in oracle.linear_grad.NAMES]
    y_t = oracle.linear_branch_torch(*ts, S, 2, 1, rule, 0.5, 0.5, 1e-6).numpy()
    np.testing.assert_allclose(y_t, y_np, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("rule,radius,text", [
    ("vdn_solve", 0, True), ("vdn_solve", 1, False), ("vdn_scaled", 0, True),
    ("sana_scaled", 0, True)])
def test_grad_matches_central_differences(rule, radius, text):
    # radius 0 with 6 frames in chunks of 2 leaves a far field on both sides
    # of every window, so every input reaches y through the linear branch
    x = _case(61 + radius, text=text)
    S = 3
    rng = np.random.default_rng(62)
    g = rng.standard_normal(x["q"].shape)
    names = oracle.linear_grad.NAMES

    def loss(xx):
        y, _ = oracle.linear_branch(*(xx[n] for n in names), S, 2, radius, rule, 0.5, 0.5,
                                    1e-6)
        return float((y * g).sum())

    grads = oracle.linear_branch_grad(*(x[n] for n in names), g, S, 2, radius, rule)
    h = 1e-6
    for n in names:
        if x[n] is None:
            continue
        a = np.array(x[n], dtype=np.float64)
        num = np.empty_like(a)
        for idx in np.ndindex(*a.shape):
            old = a[idx]
            a[idx] = old + h
            up = loss({**x, n: a})
            a[idx] = old - h
            dn = loss({**x, n: a})
            a[idx] = old
            num[idx] = (up - dn) / (2 * h)
        scale = max(np.abs(num).max(), 1e-3)
        assert np.abs(grads[n] - num).max() <= 1e-6 * scale, (n, np.abs(grads[n] - num).max())
        assert np.abs(grads[n]).max() > 0.0, n
