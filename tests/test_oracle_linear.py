"""Pins of the oracle's linear branch (CPU only).

Steps follow the VDN-H3 article: "Step 1: NoPE features", "Step 2: per-frame
statistics A, B", "Step 3: delta-rule state update" (rules table), "Step 4:
bidirectional scan + boundary gather", "Step 5: readout and gating" and "Text
state". Each test checks the oracle against something other than itself: a
hand-worked example, a closed form, an invariant, a library routine or exact
rational arithmetic.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.signal

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(2024)


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- features
def test_silu_closed_forms():
    x = np.linspace(-30, 30, 601)
    s = oracle.silu(x)
    assert s[300] == 0.0                                    # silu(0) = 0
    # x sigmoid(x) - (-x) sigmoid(-x) = x (sigmoid(x) + sigmoid(-x)) = x
    assert np.abs(s - oracle.silu(-x) - x).max() < 1e-12
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
    assert np.abs(oracle.silu(np.array([40.0])) - 40.0).max() < 1e-12


def test_short_conv_identity_and_lfilter():
    F, S, d = 3, 7, 5
    x = RNG.standard_normal((F * S, d))
    ident = np.zeros((d, 4))
    ident[:, 0] = 1.0
    assert np.array_equal(oracle.short_conv(x, ident, S), x)
    taps = RNG.standard_normal((d, 4))
    got = oracle.short_conv(x, taps, S)
    for f in range(F):
        for c in range(d):
            # causal FIR within the frame, zero history at the frame start
            ref = scipy.signal.lfilter(taps[c], [1.0], x[f * S:(f + 1) * S, c])
            assert np.abs(got[f * S:(f + 1) * S, c] - ref).max() < 1e-12
    # a frame shorter than the filter
    x2 = RNG.standard_normal((4 * 2, d))
    got2 = oracle.short_conv(x2, taps, 2)
    for f in range(4):
        for c in range(d):
            ref = scipy.signal.lfilter(taps[c], [1.0], x2[f * 2:(f + 1) * 2, c])
            assert np.abs(got2[f * 2:(f + 1) * 2, c] - ref).max() < 1e-12


def test_features_unit_norm_and_raw_q():
    S, d = 6, 8
    q, k, v = (RNG.standard_normal((4 * S, d)) for _ in range(3))
    taps = RNG.standard_normal((d, 4)) * 0.5
    qh, kh, vh = oracle.features(q, k, v, taps, taps, S)
    assert np.abs(np.linalg.norm(qh, axis=1) - 1).max() < 1e-14
    assert np.abs(np.linalg.norm(kh, axis=1) - 1).max() < 1e-14
    # q is not convolved: q^ is L2(SiLU(q)) token by token
    sq = q / (1 + np.exp(-q))
    assert np.abs(qh - sq / np.linalg.norm(sq, axis=1, keepdims=True)).max() < 1e-14
    # v gets the conv only (no activation): linear in v
    _, _, vh2 = oracle.features(q, k, 2.0 * v, taps, taps, S)
    assert np.abs(vh2 - 2.0 * vh).max() < 1e-13


def test_l2_clamp_zero_and_tiny_rows():
    # "Step 1" L2 with the epsilon reading x / max(||x||, 1e-12): a zero row
    # stays zero (no 0/0), a row of norm 5e-13 is divided by 1e-12, not by its
    # norm, and a row of norm exactly 1e-12 by that norm (both sides agree)
    x = np.array([[0.0, 0.0, 0.0],
                  [3e-13, 4e-13, 0.0],
                  [6e-13, 0.0, 8e-13],
                  [3.0, 0.0, 4.0]])
    got = oracle.l2_normalize(x)
    assert np.array_equal(got[0], np.zeros(3))
    assert np.allclose(got[1], [0.3, 0.4, 0.0], rtol=1e-12, atol=0)
    assert np.allclose(got[2], [0.6, 0.0, 0.8], rtol=1e-12, atol=0)
    assert np.allclose(got[3], [0.6, 0.0, 0.8], rtol=1e-15, atol=0)
    # a different eps moves only the clamped rows
    got2 = oracle.l2_normalize(x, eps=1e-13)
    assert np.allclose(got2[1], [0.6, 0.8, 0.0], rtol=1e-12, atol=0)
    assert np.array_equal(got2[3], got[3])
    # the features of an all-zero k row (SiLU(0) = 0) are zero, so such a
    # token adds nothing to A and B whatever its beta
    S, d = 4, 5
    k = RNG.standard_normal((S, d))
    k[2] = 0.0
    taps = np.zeros((d, 4))
    taps[:, 0] = 1.0
    _, kh, vh = oracle.features(k, k, k, taps, taps, S)
    assert np.array_equal(kh[2], np.zeros(d))
    A, B = oracle.frame_statistics(kh, vh, np.array([0.5, 0.7, 1e6, 0.2]), S)
    keep = [0, 1, 3]
    A2, B2 = oracle.frame_statistics(kh[keep], vh[keep], np.array([0.5, 0.7, 0.2]), 3)
    assert np.allclose(A, A2, rtol=1e-13, atol=1e-15)
    assert np.allclose(B, B2, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- statistics
def test_statistics_invariants_and_bruteforce():
    S, d, F = 9, 6, 3
    kh = oracle.l2_normalize(RNG.standard_normal((F * S, d)))
    vh = RNG.standard_normal((F * S, d))
    beta = RNG.random(F * S)
    A, B = oracle.frame_statistics(kh, vh, beta, S)
    for f in range(F):
        assert np.abs(A[f] - A[f].T).max() < 1e-15
        assert np.linalg.eigvalsh(A[f]).min() > -1e-12
        # unit keys: tr(A_f) = sum of beta over the frame
        assert abs(np.trace(A[f]) - beta[f * S:(f + 1) * S].sum()) < 1e-12
        for i in range(d):
            for j in range(d):
                a = sum(beta[n] * kh[n, i] * kh[n, j] for n in range(f * S, (f + 1) * S))
                b = sum(beta[n] * vh[n, i] * kh[n, j] for n in range(f * S, (f + 1) * S))
                assert abs(A[f, i, j] - a) < 1e-12 and abs(B[f, i, j] - b) < 1e-12


# ---------------------------------------------------------------- rules
@pytest.mark.parametrize("rule", oracle.RULES)
def test_rules_hand_worked_2x2(rule):
    g = _gold("rules_2x2.json")
    k, v = np.array(g["k"]), np.array(g["v"])
    A, B = oracle.frame_statistics(k[None], v[None], np.array([g["beta"]]), 1)
    assert np.abs(A[0] - np.array(g["A"])).max() < 1e-15
    assert np.abs(B[0] - np.array(g["B"])).max() < 1e-15
    out = oracle.rule_step(np.array(g["S_in"]), A[0], B[0], np.array(g["alpha"]),
                           rule, g["c"])
    assert np.abs(out - np.array(g[rule])).max() < 1e-14


def _spd_case(d=7, n=11):
    k = oracle.l2_normalize(RNG.standard_normal((n, d)))
    v = RNG.standard_normal((n, d))
    beta = RNG.random(n)
    A, B = oracle.frame_statistics(k, v, beta, n)
    return A[0], B[0], RNG.standard_normal((d, d)), RNG.uniform(0.5, 1.0, d)


def test_solve_residual():
    A, B, S, al = _spd_case()
    I = np.eye(A.shape[0])
    for rule, c, M, cb in (("vdn_solve", 1.0, I + A, 1.0),
                           ("vdn_scaled", 0.37, I + 0.37 ** 2 * A, 0.37)):
        X = oracle.rule_step(S, A, B, al, rule, c)
        rhs = S * al[None, :] + cb * B
        assert np.linalg.norm(X @ M - rhs) / np.linalg.norm(rhs) < 1e-13


def test_sherman_morrison_single_token():
    d = 6
    k = oracle.l2_normalize(RNG.standard_normal((1, d)))[0]
    v = RNG.standard_normal(d)
    beta = 0.73
    S, al = RNG.standard_normal((d, d)), RNG.uniform(0.5, 1, d)
    A, B = oracle.frame_statistics(k[None], v[None], np.array([beta]), 1)
    got = oracle.rule_step(S, A[0], B[0], al, "vdn_solve")
    # (I + beta k k^T)^-1 = I - beta/(1+beta) k k^T for a unit k
    inv = np.eye(d) - beta / (1 + beta) * np.outer(k, k)
    ref = (S * al + beta * np.outer(v, k)) @ inv
    assert np.abs(got - ref).max() < 1e-13


def test_vdn_scaled_c1_is_vdn_solve_and_beta0():
    A, B, S, al = _spd_case()
    a = oracle.rule_step(S, A, B, al, "vdn_solve")
    b = oracle.rule_step(S, A, B, al, "vdn_scaled", 1.0)
    assert np.abs(a - b).max() < 1e-13
    Z = np.zeros_like(A)
    for rule in oracle.RULES:
        assert np.abs(oracle.rule_step(S, Z, Z, al, rule, 0.5) - S * al).max() < 1e-15


def test_sana_is_first_order_truncation():
    # vdn_scaled - sana_scaled = -c^3 B A + O(c^4): slope 3 in log-log
    A, B, S, al = _spd_case()
    cs = np.array([0.02, 0.01, 0.005])
    gaps = [np.linalg.norm(oracle.rule_step(S, A, B, al, "vdn_scaled", c)
                           - oracle.rule_step(S, A, B, al, "sana_scaled", c)) for c in cs]
    slope = np.polyfit(np.log(cs), np.log(gaps), 1)[0]
    assert abs(slope - 3.0) < 0.1
    assert abs(gaps[-1] / cs[-1] ** 3 / np.linalg.norm(B @ A) - 1) < 0.05


# ---------------------------------------------------------------- scan
def _scan_case(F=9, d=5, S=4, beta_zero=False):
    kh = oracle.l2_normalize(RNG.standard_normal((F * S, d)))
    vh = RNG.standard_normal((F * S, d))
    beta = np.zeros(F * S) if beta_zero else RNG.random(F * S)
    A, B = oracle.frame_statistics(kh, vh, beta, S)
    alpha = RNG.uniform(0.8, 1.0, (F, d))
    return A, B, alpha, RNG.standard_normal((d, d))


@pytest.mark.parametrize("rule", oracle.RULES)
def test_scan_frame_reversal(rule):
    A, B, al, S0 = _scan_case()
    P, Q = oracle.scan(A, B, al, S0, rule, 0.5)
    Pr, Qr = oracle.scan(A[::-1], B[::-1], al[::-1], S0, rule, 0.5)
    # prefix of the reversed video == reversed suffix of the original
    assert np.abs(Pr - Q[::-1]).max() < 1e-12 * max(1, np.abs(Q).max())
    assert np.abs(Qr - P[::-1]).max() < 1e-12 * max(1, np.abs(P).max())


@pytest.mark.parametrize("rule", oracle.RULES)
def test_scan_associative_recomputation(rule):
    # every rule is an affine map S -> S G_f + C_f; composing the maps in a
    # balanced tree must give the same states as the frame loop
    A, B, al, S0 = _scan_case(F=8)
    c = 0.5
    d = A.shape[1]
    I = np.eye(d)
    maps = []
    for f in range(A.shape[0]):
        if rule == "sana_scaled":
            G, C = np.diag(al[f]) @ (I - c * c * A[f]), c * B[f]
        else:
            cc, cb = (1.0, 1.0) if rule == "vdn_solve" else (c, c)
            M = np.linalg.inv(I + cc * cc * A[f])
            G, C = np.diag(al[f]) @ M, cb * B[f] @ M
        maps.append((G, C))

    def compose(m1, m2):  # apply m1 then m2
        return m1[0] @ m2[0], m1[1] @ m2[0] + m2[1]

    def tree(ms):
        if len(ms) == 1:
            return ms[0]
        h = len(ms) // 2
        return compose(tree(ms[:h]), tree(ms[h:]))

    P, Q = oracle.scan(A, B, al, S0, rule, c)
    G, C = tree(maps)
    assert np.linalg.norm(S0 @ G + C - P[-1]) / np.linalg.norm(P[-1]) < 1e-10
    G, C = tree(maps[::-1])
    assert np.linalg.norm(S0 @ G + C - Q[0]) / np.linalg.norm(Q[0]) < 1e-10
    G, C = tree(maps[:5])
    assert np.linalg.norm(S0 @ G + C - P[5]) / np.linalg.norm(P[5]) < 1e-10


# ---------------------------------------------------------------- gather/readout
def test_gather_beta0_closed_form_and_halves():
    F, d, chunk, radius = 13, 4, 3, 1
    A = np.zeros((F, d, d))
    alpha = RNG.uniform(0.8, 1.0, (F, d))
    S_text = RNG.standard_normal((d, d))
    scale = _gold("page_facts.json")["text_state"]["scale"]
    P, Q = oracle.scan(A, A, alpha, scale * S_text, "vdn_solve")
    lo, hi = oracle.window_bounds(F, chunk, radius)
    for t in range(F):
        St = oracle.gathered_state(P, Q, alpha, lo, hi, t)
        ref = scale * S_text * (np.prod(alpha[:t + 1], axis=0) + np.prod(alpha[t:], axis=0))
        assert np.abs(St - ref).max() < 1e-13
    ones = np.ones((F, d))
    P, Q = oracle.scan(A, A, ones, scale * S_text, "vdn_solve")
    halves = _gold("page_facts.json")["text_state"]["halves_sum"]
    for t in range(F):
        assert np.abs(oracle.gathered_state(P, Q, ones, lo, hi, t) - halves * S_text).max() < 1e-14


def test_readout_norm_gate_and_zero():
    d, n = 16, 5
    S_t = RNG.standard_normal((d, d))
    qh = oracle.l2_normalize(RNG.standard_normal((n, d)))
    w = np.ones(d)
    y = oracle.readout(S_t, qh, np.zeros((n, d)), w, eps=1e-6)
    # gate pre-activation 0 -> sigmoid = 1/2; RMSNorm output has RMS 1 (up to eps)
    rms = np.sqrt((y * y).mean(axis=1))
    assert np.abs(rms - 0.5).max() < 1e-5
    o = qh @ S_t.T
    assert np.abs(y - 0.5 * o / np.sqrt((o * o).mean(axis=1, keepdims=True) + 1e-6)).max() < 1e-14
    assert not np.any(oracle.readout(np.zeros((d, d)), qh, RNG.standard_normal((n, d)), w))
    # huge states (a diverging sana_scaled scan) normalise without overflow
    yb = oracle.readout(S_t * 1e200, qh, np.zeros((n, d)), w, eps=1e-6)
    assert np.isfinite(yb).all() and np.abs(yb - y).max() < 1e-5


# ---------------------------------------------------------------- exact rational
def _frac_inv(M):
    n = len(M)
    a = [row[:] + [Fraction(int(i == j)) for j in range(n)] for i, row in enumerate(M)]
    for col in range(n):
        piv = next(r for r in range(col, n) if a[r][col] != 0)
        a[col], a[piv] = a[piv], a[col]
        p = a[col][col]
        a[col] = [x / p for x in a[col]]
        for r in range(n):
            if r != col and a[r][col] != 0:
                fct = a[r][col]
                a[r] = [x - fct * y for x, y in zip(a[r], a[col])]
    return [row[n:] for row in a]


def _mm(X, Y):
    return [[sum(X[i][k] * Y[k][j] for k in range(len(Y))) for j in range(len(Y[0]))]
            for i in range(len(X))]


@pytest.mark.parametrize("rule", oracle.RULES)
def test_linear_branch_exact_rational(rule):
    """Statistics -> scans -> gather -> readout pre-norm, recomputed in exact
    rational arithmetic from the oracle's own fp64 features (converted
    exactly), then compared with the fp64 pipeline."""
    F, S, d, chunk, radius, c = 7, 2, 3, 2, 0, Fraction(1, 2)
    q, k, v = (RNG.standard_normal((F * S, d)) for _ in range(3))
    taps = RNG.standard_normal((d, 4)) * 0.5
    beta = RNG.random(F * S)
    alpha = RNG.uniform(0.8, 1.0, (F, d))
    S_text = RNG.standard_normal((d, d))
    gate = np.zeros((F * S, d))
    y, inter = oracle.linear_branch(q, k, v, beta, alpha, gate, S_text, taps, taps,
                                    np.ones(d), S, chunk, radius, rule, 0.5, 0.5,
                                    1e-6, keep=True)
    qh, kh, vh = inter["qh"], inter["kh"], inter["vh"]
    Fr = lambda x: Fraction(float(x))  # noqa: E731 exact conversion
    I = [[Fraction(int(i == j)) for j in range(d)] for i in range(d)]
    As, Bs = [], []
    for f in range(F):
        A = [[sum(Fr(beta[n]) * Fr(kh[n, i]) * Fr(kh[n, j]) for n in range(f * S, (f + 1) * S))
              for j in range(d)] for i in range(d)]
        B = [[sum(Fr(beta[n]) * Fr(vh[n, i]) * Fr(kh[n, j]) for n in range(f * S, (f + 1) * S))
              for j in range(d)] for i in range(d)]
        As.append(A)
        Bs.append(B)

    def step(Sm, f):
        SD = [[Sm[i][j] * Fr(alpha[f, j]) for j in range(d)] for i in range(d)]
        A, B = As[f], Bs[f]
        if rule == "vdn_solve":
            M = _frac_inv([[I[i][j] + A[i][j] for j in range(d)] for i in range(d)])
            return _mm([[SD[i][j] + B[i][j] for j in range(d)] for i in range(d)], M)
        if rule == "vdn_scaled":
            M = _frac_inv([[I[i][j] + c * c * A[i][j] for j in range(d)] for i in range(d)])
            return _mm([[SD[i][j] + c * B[i][j] for j in range(d)] for i in range(d)], M)
        T = _mm(SD, [[I[i][j] - c * c * A[i][j] for j in range(d)] for i in range(d)])
        return [[T[i][j] + c * B[i][j] for j in range(d)] for i in range(d)]

    S0 = [[Fraction(1, 2) * Fr(S_text[i, j]) for j in range(d)] for i in range(d)]
    P = [S0]
    for f in range(F):
        P.append(step(P[-1], f))
    Q = [None] * (F + 1)
    Q[F] = S0
    for f in range(F - 1, -1, -1):
        Q[f] = step(Q[f + 1], f)
    lo, hi = oracle.window_bounds(F, chunk, radius)
    for t in range(F):
        a = [Fraction(1)] * d
        b = [Fraction(1)] * d
        for j in range(lo[t], t + 1):
            a = [a[i] * Fr(alpha[j, i]) for i in range(d)]
        for j in range(t, hi[t] + 1):
            b = [b[i] * Fr(alpha[j, i]) for i in range(d)]
        St = [[P[lo[t]][i][j] * a[j] + Q[hi[t] + 1][i][j] * b[j] for j in range(d)]
              for i in range(d)]
        Stf = np.array([[float(x) for x in row] for row in St])
        assert np.abs(Stf - inter["states"][t]).max() <= 1e-12 * max(1.0, np.abs(Stf).max())
        for n in range(t * S, (t + 1) * S):
            o = np.array([float(sum(St[i][j] * Fr(qh[n, j]) for j in range(d))) for i in range(d)])
            ref = 0.5 * o / np.sqrt((o * o).mean() + 1e-6)
            assert np.abs(y[n] - ref).max() < 1e-12


# ---------------------------------------------------------------- text state
def test_text_state_single_token_closed_form():
    d = 8
    k = RNG.standard_normal((1, d))
    v = RNG.standard_normal((1, d))
    beta = np.array([0.6])
    got = oracle.text_state(k, v, beta)
    kh = oracle.l2_normalize(oracle.silu(k))[0]
    # Sherman-Morrison with a unit key: B (I + A)^-1 = beta/(1+beta) v k^T
    assert np.abs(got - 0.6 / 1.6 * np.outer(v[0], kh)).max() < 1e-14


# ---------------------------------------------------------------- alpha producer
def test_frame_alpha_closed_forms_and_bruteforce():
    # the gate reading alpha_f = exp(-exp(a) softplus(mean_f(k) W + b))
    S, d, F = 7, 5, 4
    k = RNG.standard_normal((F * S, d))
    a_log = RNG.standard_normal(d) * 0.5
    # W = 0, b = 0: softplus(0) = ln 2, so alpha = 2^(-exp(a)) for every frame
    got = oracle.frame_alpha(k, np.zeros((d, d)), np.zeros(d), a_log, S)
    assert np.allclose(got, np.broadcast_to(2.0 ** -np.exp(a_log), (F, d)), rtol=1e-14, atol=0)
    # exp(a) = 1 and z = 0: alpha = 1/2 exactly
    half = oracle.frame_alpha(k, np.zeros((d, d)), np.zeros(d), np.zeros(d), S)
    assert np.allclose(half, 0.5, rtol=1e-15, atol=0)
    # scalar brute force with an unsymmetric W (input channel i, output j)
    w = RNG.standard_normal((d, d))
    assert not np.allclose(w, w.T)
    b = RNG.standard_normal(d)
    got = oracle.frame_alpha(k, w, b, a_log, S)
    for f in range(F):
        m = [sum(k[f * S + s, i] for s in range(S)) / S for i in range(d)]
        for j in range(d):
            z = sum(m[i] * w[i, j] for i in range(d)) + b[j]
            sp = max(z, 0.0) + math.log1p(math.exp(-abs(z)))
            ref = math.exp(-math.exp(a_log[j]) * sp)
            assert abs(got[f, j] - ref) <= 1e-13 * ref
    # range and monotonicity: a larger pre-activation gives a smaller gate
    assert np.all((got > 0) & (got < 1))
    up = oracle.frame_alpha(k, w, b + 1.0, a_log, S)
    assert np.all(up < got)
    far = oracle.frame_alpha(k, w, b - 60.0, a_log, S)
    assert np.all(1.0 - far < 1e-20) and np.all(far <= 1.0)
    # the order of tokens inside a frame does not matter; frames are separate
    perm = np.concatenate([f * S + RNG.permutation(S) for f in range(F)])
    assert np.allclose(oracle.frame_alpha(k[perm], w, b, a_log, S), got, rtol=1e-13, atol=0)
    k2 = k.copy()
    k2[S:2 * S] += 1.0
    got2 = oracle.frame_alpha(k2, w, b, a_log, S)
    assert np.array_equal(got2[[0, 2, 3]], got[[0, 2, 3]]) and not np.allclose(got2[1], got[1])
