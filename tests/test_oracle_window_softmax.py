"""Pins of the oracle's window geometry and softmax branch (CPU only).

Window geometry: VDN-H3 article, "What the far field outside the window is";
partition: "Step 4: bidirectional scan + boundary gather".
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_window_golden_examples():
    for case in _gold("window_examples.json")["cases"]:
        lo, hi = oracle.window_bounds(case["frames"], case["chunk"], case["radius"])
        if "lo" in case:
            assert lo.tolist() == case["lo"]
            assert hi.tolist() == case["hi"]
        else:
            t = case["t"]
            assert (lo[t], hi[t]) == (case["lo_t"], case["hi_t"])


def test_window_page_facts():
    facts = _gold("page_facts.json")["window"]
    F = facts["example_video_frames"]
    lo, hi = oracle.window_bounds(F, facts["chunk"], facts["radius"])
    widths = hi - lo + 1
    # a middle frame sees about 15 frames; interior windows are exactly 15
    assert widths[F // 2] == facts["middle_frame_window_frames"]
    interior = [t for t in range(F) if facts["chunk"] <= t < F - facts["chunk"]]
    assert all(widths[t] == 15 for t in interior)
    # most frames of a 100-frame video lie outside every middle frame's window
    assert F - widths[F // 2] > F // 2


@pytest.mark.parametrize("F", range(1, 41))
def test_window_bruteforce_and_partition(F):
    for chunk in range(1, 8):
        for radius in range(0, 4):
            lo, hi = oracle.window_bounds(F, chunk, radius)
            for t in range(F):
                seen = [u for u in range(F) if abs(u // chunk - t // chunk) <= radius]
                assert seen == list(range(seen[0], seen[-1] + 1))
                assert (lo[t], hi[t]) == (seen[0], seen[-1])
                # prefix [0, lo-1], window [lo, hi], suffix [hi+1, F-1]:
                # disjoint and covering every frame exactly once
                parts = list(range(0, lo[t])) + list(range(lo[t], hi[t] + 1)) \
                    + list(range(hi[t] + 1, F))
                assert parts == list(range(F))
                assert lo[t] <= t <= hi[t]


def _bruteforce_masked(q, k, v, S, chunk, radius):
    """N x N masked softmax written out in Python scalars (tiny inputs)."""
    N, d = q.shape
    out = np.zeros((N, v.shape[1]))
    for n in range(N):
        tn = n // S
        keys = [m for m in range(N) if abs((m // S) // chunk - tn // chunk) <= radius]
        sc = [sum(float(q[n, i]) * float(k[m, i]) for i in range(d)) / math.sqrt(d) for m in keys]
        mx = max(sc)
        e = [math.exp(s - mx) for s in sc]
        z = sum(e)
        for j, m in enumerate(keys):
            out[n] += (e[j] / z) * v[m]
    return out


@pytest.mark.parametrize("F,S,d,chunk,radius", [(7, 3, 4, 2, 1), (9, 2, 3, 3, 0), (6, 4, 5, 5, 1)])
def test_softmax_bruteforce(F, S, d, chunk, radius):
    rng = np.random.default_rng(11)
    N = F * S
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    lo, hi = oracle.window_bounds(F, chunk, radius)
    got = oracle.softmax_branch(q, k, v, S, lo, hi)
    ref = _bruteforce_masked(q, k, v, S, chunk, radius)
    assert np.abs(got - ref).max() < 1e-12
    rows = [0, N // 2, N - 1]
    assert np.abs(oracle.softmax_rows(q, k, v, S, lo, hi, rows) - ref[rows]).max() < 1e-12


def test_softmax_full_attention_reduces_to_sdpa():
    rng = np.random.default_rng(12)
    F, S, d, chunk = 8, 5, 16, 2
    N = F * S
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    lo, hi = oracle.window_bounds(F, chunk, radius=F)  # window covers everything
    assert (lo == 0).all() and (hi == F - 1).all()
    got = oracle.softmax_branch(q, k, v, S, lo, hi)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x)[None, None] for x in (q, k, v)))[0, 0].numpy()
    assert np.abs(got - ref).max() < 1e-12


def test_softmax_radius0_is_block_diagonal():
    rng = np.random.default_rng(13)
    F, S, d, chunk = 7, 4, 8, 3
    N = F * S
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    lo, hi = oracle.window_bounds(F, chunk, radius=0)
    got = oracle.softmax_branch(q, k, v, S, lo, hi)
    for c0 in range(0, F, chunk):
        sl = slice(c0 * S, min(F, c0 + chunk) * S)
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(x[sl])[None, None] for x in (q, k, v)))[0, 0].numpy()
        assert np.abs(got[sl] - ref).max() < 1e-12
