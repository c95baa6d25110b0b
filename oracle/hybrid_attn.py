"""Plain fp64 definition of the VDN-H3 hybrid attention forward.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import this module.

The method is the one the VDN-H3 article ("VDN-Minimax-H3", icman.com.cn news
81972) describes: a chunk-aligned windowed softmax over latent frames plus a
bidirectional delta-rule linear branch for every frame outside the window.
Section names below are those of that article (English glosses):

* "Why video models are stuck on attention" -- the two branches share one
  q/k/v and their outputs are summed.
* "What the far field outside the window is" -- chunk = 5 latent frames, one
  chunk on each side (radius 1), window bounds per query frame.
* "Step 1: NoPE features" -- short conv on k and v only, SiLU, L2 on q and k.
* "Step 2: per-frame statistics A, B" -- A = sum k beta k^T, B = sum v beta k^T.
* "Step 3: delta-rule state update" -- vdn_solve and the rules table
  (sana_scaled, vdn_scaled).
* "Step 4: bidirectional scan + boundary gather" -- prefix/suffix states,
  prefix[lo-1] and suffix[hi+1], alpha bridge decay.
* "Step 5: readout and gating" -- query readout, RMSNorm, output gate.
* "Text state" -- both scans start from 0.5 x the text state.

The article drops the '=' and '+' signs of its formulas in extraction; they are
read back as '=' and '+' (the only reading under which sana_scaled is the
first-order truncation of vdn_scaled, as the rules table says).

Everything is numpy float64. Inputs of lower precision are upcast exactly.
Tokens are frame-major: token n belongs to frame n // S.
"""

from __future__ import annotations

import math

import numpy as np

RULES = ("vdn_solve", "sana_scaled", "vdn_scaled")

_F64 = np.float64


# --------------------------------------------------------------------------
# Window geometry
# --------------------------------------------------------------------------
def window_bounds(frames: int, chunk: int, radius: int):
    """Inclusive key-frame window [lo_t, hi_t] of every query frame t.

    Follows "What the far field outside the window is": frames are grouped in
    chunks of ``chunk`` latent frames counted from frame 0; a query frame sees
    its own chunk and ``radius`` chunks on each side, clipped to the video.
    The last chunk may be partial.

    Pinned by: brute-force enumeration of chunk distances, the exact
    prefix/window/suffix partition of "Step 4", and the article's "about 15
    frames" for a middle frame at chunk 5, radius 1.
    """
    if frames <= 0 or chunk <= 0 or radius < 0:
        raise ValueError("frames, chunk must be > 0 and radius >= 0")
    lo = np.empty(frames, dtype=np.int32)
    hi = np.empty(frames, dtype=np.int32)
    for t in range(frames):
        c = t // chunk
        lo[t] = max(0, (c - radius) * chunk)
        hi[t] = min(frames - 1, (c + radius + 1) * chunk - 1)
    return lo, hi


# --------------------------------------------------------------------------
# Softmax branch
# --------------------------------------------------------------------------
def _softmax_block(qs, ks, vs):
    """Row softmax(qs ks^T / sqrt(d)) @ vs, max-subtracted, in fp64."""
    d = qs.shape[1]
    s = (qs @ ks.T) / math.sqrt(d)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vs


def softmax_branch(q, k, v, S: int, lo, hi, row_block: int = 512, frames=None):
    """Windowed softmax output for one (batch, head) slice.

    q, k, v: [N, d] (the softmax branch's q/k, i.e. RoPE'd ones if the caller
    has them). Query token n in frame t attends to every token of frames
    lo_t..hi_t with scale 1/sqrt(d), no bias and no causal mask ("Why video
    models are stuck on attention", "What the far field outside the window
    is"). Query rows are processed ``row_block`` at a time only to bound
    memory; each row's arithmetic is the plain definition.

    ``frames``: optional (t0, t1); then only the query frames t0..t1-1 are
    computed and the result holds their rows, [(t1 - t0) * S, d].

    Pinned by: a brute-force N x N masked softmax, textbook full attention
    (radius covering all chunks) and chunk-block-diagonal attention (radius 0).
    """
    q = np.asarray(q, _F64)
    k = np.asarray(k, _F64)
    v = np.asarray(v, _F64)
    N, d = q.shape
    t0, t1 = (0, N // S) if frames is None else frames
    out = np.empty(((t1 - t0) * S, v.shape[1]), dtype=_F64)
    for t in range(t0, t1):
        k0, k1 = int(lo[t]) * S, (int(hi[t]) + 1) * S
        for r0 in range(t * S, (t + 1) * S, row_block):
            r1 = min((t + 1) * S, r0 + row_block)
            out[r0 - t0 * S:r1 - t0 * S] = _softmax_block(q[r0:r1], k[k0:k1], v[k0:k1])
    return out


def softmax_rows(q, k, v, S: int, lo, hi, rows):
    """Windowed softmax output for the selected query ``rows`` only.

    Same definition as :func:`softmax_branch`, one query row at a time; used
    for sampled checks at sizes where the full branch is too slow on a CPU.
    """
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), v.shape[1]), dtype=_F64)
    for i, n in enumerate(rows):
        t = int(n) // S
        k0, k1 = int(lo[t]) * S, (int(hi[t]) + 1) * S
        out[i] = _softmax_block(np.asarray(q[n:n + 1], _F64),
                                np.asarray(k[k0:k1], _F64),
                                np.asarray(v[k0:k1], _F64))[0]
    return out


# --------------------------------------------------------------------------
# Step 1: NoPE features
# --------------------------------------------------------------------------
def silu(x):
    """SiLU x * sigmoid(x) = x / (1 + exp(-x)), elementwise ("Step 1")."""
    x = np.asarray(x, _F64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def l2_normalize(x, eps: float = 1e-12):
    """x / max(||x||_2, eps) along the last axis ("Step 1": L2 on q and k)."""
    x = np.asarray(x, _F64)
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def short_conv(x, taps, S: int):
    """Depthwise causal width-4 conv along each frame's token order.

    "Step 1" names a separable short conv applied to k and v only. Read as a
    per-channel (depthwise) causal filter over the tokens of one frame:
    y[s, c] = sum_j taps[c, j] * x[s - j, c] for j = 0..3, where tokens before
    the frame's first token count as zero (no crossing of frame boundaries) and
    tap 0 multiplies the current token. No bias.

    Pinned by: identity taps (1, 0, 0, 0) and scipy.signal.lfilter per channel.
    """
    x = np.asarray(x, _F64)
    taps = np.asarray(taps, _F64)
    N, d = x.shape
    F = N // S
    width = taps.shape[1]
    xf = x.reshape(F, S, d)
    y = np.zeros_like(xf)
    for j in range(width):
        if j >= S:
            break
        y[:, j:, :] += taps[:, j] * xf[:, : S - j, :]
    return y.reshape(N, d)


def features(q, k, v, conv_k, conv_v, S: int):
    """NoPE features of "Step 1": q^ = L2(SiLU(q)), k^ = L2(SiLU(conv_k(k))),
    v^ = conv_v(v). q keeps its raw pre-RoPE value; v gets no activation.

    Pinned by: unit norms of q^, k^; identity conv; SiLU closed form.
    """
    qh = l2_normalize(silu(q))
    kh = l2_normalize(silu(short_conv(k, conv_k, S)))
    vh = short_conv(v, conv_v, S)
    return qh, kh, vh


# --------------------------------------------------------------------------
# Step 2: per-frame statistics
# --------------------------------------------------------------------------
def frame_statistics(kh, vh, beta, S: int):
    """A_f = sum_{n in f} beta_n k^_n k^_n^T and B_f = sum beta_n v^_n k^_n^T.

    "Step 2" compresses the S tokens of a frame into two d x d matrices; the
    sum (not the mean) is taken, as written there. B is d_v x d_k.

    Pinned by: symmetry and PSD of A, tr(A_f) = sum beta (unit k^), a
    token-by-token brute-force re-sum, and an exact rational re-computation.
    """
    kh = np.asarray(kh, _F64)
    vh = np.asarray(vh, _F64)
    beta = np.asarray(beta, _F64)
    N, d = kh.shape
    F = N // S
    A = np.empty((F, d, d), dtype=_F64)
    B = np.empty((F, vh.shape[1], d), dtype=_F64)
    for f in range(F):
        sl = slice(f * S, (f + 1) * S)
        kb = kh[sl] * beta[sl, None]
        A[f] = kb.T @ kh[sl]
        B[f] = (vh[sl] * beta[sl, None]).T @ kh[sl]
    return A, B


# --------------------------------------------------------------------------
# Step 3: update rules
# --------------------------------------------------------------------------
def rule_step(S_in, A, B, alpha, rule: str = "vdn_solve", c: float = 1.0):
    """One delta-rule state update ("Step 3" and its rules table).

    D = diag(alpha) right-multiplies the state (S is d_v x d_k, alpha is over
    the key channels):

    * vdn_solve:   S_out = (S_in D + B) (I + A)^-1
    * sana_scaled: S_out = (S_in D)(I - c^2 A) + c B
    * vdn_scaled:  S_out = (S_in D + c B)(I + c^2 A)^-1

    The inverse is applied by an LU solve (X (I + A) = rhs).

    Pinned by: solve residual, Sherman-Morrison single-token closed form,
    vdn_scaled(c=1) == vdn_solve, the c^3 gap between sana_scaled and
    vdn_scaled, beta = 0 giving S_in D, and a hand-worked 2 x 2 example.
    """
    S_in = np.asarray(S_in, _F64)
    A = np.asarray(A, _F64)
    B = np.asarray(B, _F64)
    alpha = np.asarray(alpha, _F64)
    d = A.shape[0]
    I = np.eye(d)
    SD = S_in * alpha[None, :]
    if rule == "vdn_solve":
        rhs, M = SD + B, I + A
    elif rule == "vdn_scaled":
        rhs, M = SD + c * B, I + (c * c) * A
    elif rule == "sana_scaled":
        return SD @ (I - (c * c) * A) + c * B
    else:
        raise ValueError(f"unknown rule {rule!r}")
    # X M = rhs  <=>  M^T X^T = rhs^T
    return np.linalg.solve(M.T, rhs.T).T


def frame_alpha(k, w, bias, a_log, S: int):
    """Per-frame, per-key-channel forget gate alpha_f in (0, 1) ("Step 3":
    D = diag(alpha) is a per-channel forget gate with values between 0 and 1,
    produced by a layer the article calls FrameKDAAlpha).

    The article names the producer but gives neither its formula nor its
    weights. Reading (a gate of the kind "KDA" delta-rule layers use, taken
    once per frame): pool the frame's raw k rows, project, and map through a
    decay rate,
        m_f = mean_{n in f} k_n          (d)
        z_f = m_f W + b                  (W: d x d, input channel i, output j)
        alpha_f = exp(-exp(a) * softplus(z_f)),  softplus(z) = log(1 + e^z),
    so alpha lies in (0, 1), tends to 1 where z -> -inf and falls as z grows.
    k: [N, d] (one (batch, head) slice); w: [d, d]; bias, a_log: [d].
    Returns [F, d].

    Pinned by: W = 0, b = 0 giving 2^(-exp(a)) exactly (softplus(0) = ln 2),
    a scalar brute force with an unsymmetric W (catches a transposed W), the
    range (0, 1) and monotonicity in z, and invariance to the token order
    inside a frame.
    """
    k = np.asarray(k, _F64)
    N, d = k.shape
    F = N // S
    m = k.reshape(F, S, d).mean(axis=1)
    z = m @ np.asarray(w, _F64) + np.asarray(bias, _F64)[None, :]
    softplus = np.logaddexp(0.0, z)
    return np.exp(-np.exp(np.asarray(a_log, _F64))[None, :] * softplus)


# --------------------------------------------------------------------------
# Step 4: bidirectional scan and boundary gather
# --------------------------------------------------------------------------
def scan(A, B, alpha, S0, rule: str = "vdn_solve", c: float = 1.0):
    """Prefix and suffix scans over frames ("Step 4").

    P_{-1} = S0 and P_f = R(P_{f-1}; A_f, B_f, alpha_f) for f = 0..F-1;
    Q_F = S0 and Q_f = R(Q_{f+1}; A_f, B_f, alpha_f) for f = F-1..0.
    Returns ``prefix`` [F+1, dv, dk] with prefix[i] = P_{i-1} and ``suffix``
    [F+1, dv, dk] with suffix[i] = Q_i.

    Pinned by: frame reversal (prefix of reversed frames == reversed suffix)
    and the associative recomputation through composed affine maps.
    """
    F = A.shape[0]
    prefix = np.empty((F + 1,) + tuple(S0.shape), dtype=_F64)
    suffix = np.empty_like(prefix)
    prefix[0] = S0
    for f in range(F):
        prefix[f + 1] = rule_step(prefix[f], A[f], B[f], alpha[f], rule, c)
    suffix[F] = S0
    for f in range(F - 1, -1, -1):
        suffix[f] = rule_step(suffix[f + 1], A[f], B[f], alpha[f], rule, c)
    return prefix, suffix


def gathered_state(prefix, suffix, alpha, lo, hi, t: int):
    """State read by query frame t ("Step 4", bridge mechanism).

    prefix[lo-1] holds everything left of the window and suffix[hi+1]
    everything right of it ("no overlap, no omission"). Each is multiplied by
    an alpha-determined decay across the window span. Reading: the decay runs
    from the window edge to t inclusive, a_t = prod_{j=lo..t} alpha_j and
    b_t = prod_{j=t..hi} alpha_j, applied on the key side:
    S_t = P_{lo-1} diag(a_t) + Q_{hi+1} diag(b_t).

    Pinned by: the beta = 0 closed form S_t = S0 (diag(prod_{0..t} alpha) +
    diag(prod_{t..F-1} alpha)), and with alpha = 1 the two halves of the text
    state adding up to one full prompt ("Text state").
    """
    alpha = np.asarray(alpha, _F64)
    l, h = int(lo[t]), int(hi[t])
    a = np.prod(alpha[l:t + 1], axis=0)
    b = np.prod(alpha[t:h + 1], axis=0)
    return prefix[l] * a[None, :] + suffix[h + 1] * b[None, :]


# --------------------------------------------------------------------------
# Step 5: readout and gate
# --------------------------------------------------------------------------
def _rmsnorm(o, eps: float):
    """o / sqrt(mean(o^2) + eps), computed after dividing by max|o| so that a
    diverging state (sana_scaled) cannot overflow; a zero row stays zero."""
    m = np.abs(o).max(axis=-1, keepdims=True)
    safe = np.where(m > 0, m, 1.0)
    u = o / safe
    with np.errstate(over="ignore", divide="ignore"):
        den = np.sqrt((u * u).mean(axis=-1, keepdims=True) + eps / (safe * safe))
    y = u / den
    return np.where(m > 0, y, 0.0)


def _sigmoid(g):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(g, _F64)))


def readout(S_t, qh, gate, w, eps: float = 1e-6):
    """y_n = RMSNorm(S_t q^_n) * w * sigmoid(g_n) for the tokens of one frame
    ("Step 5"). RMSNorm is over head_dim with weight w and epsilon eps; the
    output gate is a sigmoid of the gate pre-activation.

    Pinned by: RMS of the normalised readout = 1 up to eps, g = 0 giving a
    gate of 1/2, and a zero state giving exactly zero.
    """
    o = np.asarray(qh, _F64) @ np.asarray(S_t, _F64).T
    return _rmsnorm(o, eps) * np.asarray(w, _F64)[None, :] * _sigmoid(gate)


# --------------------------------------------------------------------------
# Whole branch / whole call
# --------------------------------------------------------------------------
def linear_branch(q, k, v, beta, alpha, gate, S_text, conv_k, conv_v, w, S: int,
                  chunk: int = 5, radius: int = 1, rule: str = "vdn_solve",
                  c: float = 0.5, text_scale: float = 0.5, eps: float = 1e-6,
                  keep: bool = False):
    """Bidirectional linear branch for one (batch, head) slice, steps 1-5.

    q, k, v, gate: [N, d]; beta: [N]; alpha: [F, d]; S_text: [d, d] or None;
    conv_k, conv_v: [d, 4]; w: [d]. Both scans start from text_scale * S_text
    ("Text state"), or from zero without a text state.
    Returns y [N, d] and, if ``keep``, a dict of intermediates.
    """
    N, d = np.shape(q)
    F = N // S
    lo, hi = window_bounds(F, chunk, radius)
    qh, kh, vh = features(q, k, v, conv_k, conv_v, S)
    A, B = frame_statistics(kh, vh, beta, S)
    if S_text is None:
        S0 = np.zeros((d, d), dtype=_F64)
    else:
        S0 = text_scale * np.asarray(S_text, _F64)
    prefix, suffix = scan(A, B, alpha, S0, rule, c)
    y = np.empty((N, d), dtype=_F64)
    states = np.empty((F, d, d), dtype=_F64)
    for t in range(F):
        St = gathered_state(prefix, suffix, alpha, lo, hi, t)
        states[t] = St
        sl = slice(t * S, (t + 1) * S)
        y[sl] = readout(St, qh[sl], np.asarray(gate[sl], _F64), w, eps)
    if not keep:
        return y, None
    return y, dict(lo=lo, hi=hi, qh=qh, kh=kh, vh=vh, A=A, B=B,
                   prefix=prefix, suffix=suffix, states=states)


def hybrid_attn_head(q, k, v, beta, alpha, gate, S_text, conv_k, conv_v, w,
                     S: int, chunk: int = 5, radius: int = 1,
                     rule: str = "vdn_solve", c: float = 0.5,
                     text_scale: float = 0.5, eps: float = 1e-6,
                     q_rope=None, k_rope=None, keep: bool = False):
    """Hybrid attention for one (batch, head) slice.

    out = o_sm + y: the softmax branch (RoPE'd q/k if given, else q/k) over the
    window plus the linear branch on the raw q/k/v; both read the same v
    ("Why video models are stuck on attention": shared QKV, outputs summed).
    Returns (out, o_sm, y, intermediates-or-None).
    """
    F = np.shape(q)[0] // S
    lo, hi = window_bounds(F, chunk, radius)
    qs = q if q_rope is None else q_rope
    ks = k if k_rope is None else k_rope
    o_sm = softmax_branch(qs, ks, v, S, lo, hi)
    y, inter = linear_branch(q, k, v, beta, alpha, gate, S_text, conv_k, conv_v,
                             w, S, chunk, radius, rule, c, text_scale, eps, keep)
    return o_sm + y, o_sm, y, inter


# Arguments of the whole-call tasks, set in the parent before the worker
# processes are forked (so the arrays are not pickled) and read by them.
_TASKS = {}


def _task(job):
    """One task of :func:`hybrid_attn`: ("sm", b, h, t0, t1) is the softmax
    branch of query frames t0..t1-1 of slice (b, h), ("lin", b, h) its whole
    linear branch. Returns (job, rows)."""
    a = _TASKS
    b, h = job[1], job[2]
    if job[0] == "sm":
        qs = a["q"] if a["q_rope"] is None else a["q_rope"]
        ks = a["k"] if a["k_rope"] is None else a["k_rope"]
        return job, softmax_branch(qs[b, h], ks[b, h], a["v"][b, h], a["S"], a["lo"], a["hi"],
                                   frames=(job[3], job[4]))
    st = None if a["text_state"] is None else a["text_state"][b, h]
    y, _ = linear_branch(a["q"][b, h], a["k"][b, h], a["v"][b, h], a["beta"][b, h],
                         a["alpha"][b, h], a["gate"][b, h], st, a["conv_k"][h], a["conv_v"][h],
                         a["w"], a["S"], a["chunk"], a["radius"], a["rule"], a["c"],
                         a["text_scale"], a["eps"])
    return job, y


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def hybrid_attn(q, k, v, beta, alpha, gate, text_state_, conv_k, conv_v, w,
                frames: int, S: int, chunk: int = 5, radius: int = 1,
                rule: str = "vdn_solve", c: float = 0.5,
                text_scale: float = 0.5, eps: float = 1e-6,
                q_rope=None, k_rope=None, workers: int = 1):
    """Whole call over [B, H, N, d] inputs; returns (out, o_sm, y) in fp64.

    alpha: [B, H, F, d]; beta: [B, H, N]; text_state_: [B, H, d, d] or None;
    conv_k, conv_v: [H, d, 4]; w: [d] or None (ones). Every (b, h) slice is
    the one-slice definition (:func:`hybrid_attn_head`), so out = o_sm + y
    ("Why video models are stuck on attention"). The work is cut into
    independent tasks: the softmax branch per (b, h, query chunk) -- the query
    frames of a chunk share one key range -- and the linear branch per (b, h).
    With ``workers`` > 1 the tasks run in that many forked processes, each
    with one BLAS thread; the arithmetic of a row does not depend on it.

    Pinned by: equality with :func:`hybrid_attn_head` slice by slice on a
    batch-2, two-head case with per-head conv taps, text states and alpha, in
    one process and in a pool.
    """
    Bn, H, N, d = np.shape(q)
    if N != frames * S:
        raise ValueError("N must equal frames * S")
    if w is None:
        w = np.ones(d)
    lo, hi = window_bounds(frames, chunk, radius)
    _TASKS.clear()
    _TASKS.update(q=q, k=k, v=v, beta=beta, alpha=alpha, gate=gate, text_state=text_state_,
                  conv_k=conv_k, conv_v=conv_v, w=w, S=S, chunk=chunk, radius=radius,
                  rule=rule, c=c, text_scale=text_scale, eps=eps, q_rope=q_rope,
                  k_rope=k_rope, lo=lo, hi=hi)
    jobs = [("sm", b, h, t0, min(frames, t0 + chunk))
            for b in range(Bn) for h in range(H) for t0 in range(0, frames, chunk)]
    jobs += [("lin", b, h) for b in range(Bn) for h in range(H)]
    o_sm = np.empty((Bn, H, N, d), dtype=_F64)
    y = np.empty_like(o_sm)

    def put(job, rows):
        if job[0] == "sm":
            o_sm[job[1], job[2], job[3] * S:job[4] * S] = rows
        else:
            y[job[1], job[2]] = rows

    try:
        if workers > 1:
            import multiprocessing as mp
            from concurrent.futures import ProcessPoolExecutor
            with ProcessPoolExecutor(workers, mp_context=mp.get_context("fork"),
                                     initializer=_one_blas_thread) as ex:
                for job, rows in ex.map(_task, jobs):
                    put(job, rows)
        else:
            for job in jobs:
                put(*_task(job))
    finally:
        _TASKS.clear()
    return o_sm + y, o_sm, y


def text_state(k_txt, v_txt, beta_txt):
    """Text state of one (batch, head) from T text tokens.

    The article ("Text state") starts both scans from half of a text state but
    does not spell out how that state is formed from the prompt. Reading used
    here: the text tokens form one frame of statistics with the branch's own
    feature map on k (L2(SiLU(k)), no conv: the prompt is not a token raster)
    and raw v, and the state is one vdn_solve update from zero:
    S_text = B_txt (I + A_txt)^-1.
    """
    kh = l2_normalize(silu(k_txt))
    vh = np.asarray(v_txt, _F64)
    T, d = kh.shape
    A, B = frame_statistics(kh, vh, beta_txt, T)
    return rule_step(np.zeros((vh.shape[1], d)), A[0], B[0], np.ones(d),
                     "vdn_solve", 1.0)


def rel_frobenius(x, ref):
    """||x - ref||_F / ||ref||_F in fp64; for ref == 0, 0 if x == 0 else inf."""
    x = np.asarray(x, _F64)
    ref = np.asarray(ref, _F64)
    nr = np.linalg.norm(ref.ravel())
    if nr == 0.0:
        return 0.0 if not np.any(x) else math.inf
    return float(np.linalg.norm((x - ref).ravel()) / nr)
