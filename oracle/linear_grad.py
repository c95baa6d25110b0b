"""fp64 gradient of the bidirectional delta-rule linear branch.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import this module.

The branch is the one ``hybrid_attn.linear_branch`` defines (VDN-H3 article,
"Step 1" .. "Step 5" and "Text state"): NoPE features, per-frame statistics,
prefix and suffix scans under one of the three update rules, the gathered
state with the alpha bridge decay, and the RMSNorm / sigmoid-gate readout.
Training the hybrid attention (section "Training") needs its gradient with
respect to every input. This module transcribes the same steps, one function
per step in the same order, into torch float64 operations, and takes the
gradient of L = sum(g * y) with torch autograd (the chain rule of the plain
definition; the solves are torch.linalg.solve, the products plain matmuls).

Pinned by (tests/test_oracle_linear_grad.py): its forward equals the numpy
oracle's for all three rules, and its gradient equals central finite
differences of the numpy oracle for every input tensor.
"""

from __future__ import annotations

import numpy as np
import torch

from .hybrid_attn import window_bounds

_T = torch.float64


def _silu(x):
    return x / (1.0 + torch.exp(-x))


def _l2(x, eps: float = 1e-12):
    n = torch.sqrt((x * x).sum(dim=-1, keepdim=True))
    return x / torch.clamp(n, min=eps)


def _short_conv(x, taps, S: int):
    N, d = x.shape
    xf = x.reshape(N // S, S, d)
    out = torch.zeros_like(xf)
    for j in range(taps.shape[1]):
        if j >= S:
            break
        shifted = torch.zeros_like(xf)
        shifted[:, j:, :] = xf[:, : S - j, :]
        out = out + taps[:, j] * shifted
    return out.reshape(N, d)


def _rule_step(S_in, A, B, alpha, rule: str, c: float):
    d = A.shape[0]
    eye = torch.eye(d, dtype=_T)
    SD = S_in * alpha[None, :]
    if rule == "sana_scaled":
        return SD @ (eye - (c * c) * A) + c * B
    if rule == "vdn_solve":
        rhs, M = SD + B, eye + A
    elif rule == "vdn_scaled":
        rhs, M = SD + c * B, eye + (c * c) * A
    else:
        raise ValueError(f"unknown rule {rule!r}")
    return torch.linalg.solve(M.T, rhs.T).T


def linear_branch_torch(q, k, v, beta, alpha, gate, S_text, conv_k, conv_v, w, S: int,
                        chunk: int = 5, radius: int = 1, rule: str = "vdn_solve",
                        c: float = 0.5, text_scale: float = 0.5, eps: float = 1e-6):
    """y [N, d] of the linear branch for one (batch, head) slice; every
    argument is a float64 torch tensor (S_text may be None)."""
    N, d = q.shape
    F = N // S
    lo, hi = window_bounds(F, chunk, radius)
    qh = _l2(_silu(q))
    kh = _l2(_silu(_short_conv(k, conv_k, S)))
    vh = _short_conv(v, conv_v, S)
    kf = kh.reshape(F, S, d)
    vf = vh.reshape(F, S, d)
    bf = beta.reshape(F, S, 1)
    A = torch.einsum("fsi,fsj->fij", kf * bf, kf)
    B = torch.einsum("fsi,fsj->fij", vf * bf, kf)
    S0 = torch.zeros((d, d), dtype=_T) if S_text is None else text_scale * S_text
    prefix = [S0]
    for f in range(F):
        prefix.append(_rule_step(prefix[-1], A[f], B[f], alpha[f], rule, c))
    suffix = [S0]
    for f in range(F - 1, -1, -1):
        suffix.append(_rule_step(suffix[-1], A[f], B[f], alpha[f], rule, c))
    suffix = suffix[::-1]  # suffix[i] = Q_i, suffix[F] = S0
    ys = []
    for t in range(F):
        l, h = int(lo[t]), int(hi[t])
        a = torch.prod(alpha[l:t + 1], dim=0)
        b = torch.prod(alpha[t:h + 1], dim=0)
        St = prefix[l] * a[None, :] + suffix[h + 1] * b[None, :]
        o = qh[t * S:(t + 1) * S] @ St.T
        y = o / torch.sqrt((o * o).mean(dim=-1, keepdim=True) + eps)
        ys.append(y * w[None, :] * torch.sigmoid(gate[t * S:(t + 1) * S]))
    return torch.cat(ys, dim=0)


NAMES = ("q", "k", "v", "beta", "alpha", "gate", "S_text", "conv_k", "conv_v", "w")


def linear_branch_grad(q, k, v, beta, alpha, gate, S_text, conv_k, conv_v, w, g, S: int,
                       chunk: int = 5, radius: int = 1, rule: str = "vdn_solve",
                       c: float = 0.5, text_scale: float = 0.5, eps: float = 1e-6):
    """Gradients of L = sum(g * y) with respect to every input of
    :func:`linear_branch_torch`, as a dict of numpy float64 arrays keyed by
    NAMES (``S_text`` absent when it is None). Inputs are array-likes."""
    vals = dict(q=q, k=k, v=v, beta=beta, alpha=alpha, gate=gate, S_text=S_text,
                conv_k=conv_k, conv_v=conv_v, w=w)
    ts = {n: (None if x is None else
              torch.tensor(np.asarray(x, np.float64), dtype=_T, requires_grad=True))
          for n, x in vals.items()}
    y = linear_branch_torch(*(ts[n] for n in NAMES), S, chunk, radius, rule, c, text_scale,
                            eps)
    (y * torch.tensor(np.asarray(g, np.float64), dtype=_T)).sum().backward()
    # an input y does not depend on (k, v, beta and the convs when every
    # window spans all frames) has gradient zero; autograd leaves it unset
    return {n: (t.grad.numpy() if t.grad is not None else np.zeros(tuple(t.shape)))
            for n, t in ts.items() if t is not None}
