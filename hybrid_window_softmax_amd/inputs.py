"""Seeded synthetic inputs for the hybrid attention forward.

This module draws random numbers and rounds them to the I/O dtype; it holds
none of the method's arithmetic. Both the HIP path (tests, bench) and the CPU
oracle (tests only) take their inputs from here.

Each tensor slice is drawn from ``numpy.random.default_rng([seed, tensor_id,
b, h])`` so that a slice can be regenerated on its own. Tensor ids: q 0, k 1,
v 2, gate 3, beta 4, alpha 5, text-k 6, text-v 7, text-beta 8, conv_k 9,
conv_v 10, RMSNorm weight 11 (drawn only when asked for), upstream gradient of
the softmax branch 12 (:func:`grad_output`, for the backward pass).

Distributions (the workloads of the hybrid attention on video-DiT latents):
q, k, v, gate ~ N(0, 1); beta ~ U(0, 1) per (head, token); alpha ~ U(lo, hi)
per (head, frame, key channel); conv taps ~ N(0, 1/4); RMSNorm weight = 1;
text tokens k, v ~ N(0, 1), beta ~ U(0, 1) (a workload's "beta" range, if it
gives one, replaces U(0, 1) for video and text tokens). bf16 tensors are the
fp32 draws rounded to nearest-even.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TID = dict(q=0, k=1, v=2, gate=3, beta=4, alpha=5, k_txt=6, v_txt=7,
           beta_txt=8, conv_k=9, conv_v=10, rms_weight=11, d_out=12, state=13,
           alpha_w=14, alpha_b=15, alpha_a=16, x=17, w_qkv=18, w_o=19)

# The five workloads, by name. Token counts per frame follow 832x480 (52x30
# latent grid) and 1024x1024 (64x64) canvases at 16x spatial compression.
WORKLOADS = {
    "tiny-f32": dict(name="tiny-f32", batch=1, heads=1, head_dim=16, frames=10,
            tokens_per_frame=16, dtype="f32", chunk=5, radius=1,
            rules=("vdn_solve",), c=0.5, text_tokens=0, alpha=(0.8, 1.0),
            seed=0),
    "small-bf16-text": dict(name="small-bf16-text", batch=1, heads=8, head_dim=64, frames=20,
            tokens_per_frame=256, dtype="bf16", chunk=5, radius=1,
            rules=("vdn_solve",), c=0.5, text_tokens=64, alpha=(0.8, 1.0),
            seed=1),
    "clip-832x480-31f": dict(name="clip-832x480-31f", batch=1, heads=24, head_dim=128,
            frames=31, tokens_per_frame=1560, dtype="bf16", chunk=5,
            radius=1, rules=("vdn_solve",), c=0.5, text_tokens=256,
            alpha=(0.9, 1.0), seed=2),
    "long-clip-832x480-85f": dict(name="long-clip-832x480-85f", batch=1, heads=24, head_dim=128,
            frames=85, tokens_per_frame=1560, dtype="bf16", chunk=5,
            radius=1, rules=("vdn_solve", "sana_scaled", "vdn_scaled"),
            c=0.5, text_tokens=256, alpha=(0.9, 1.0), seed=3),
    "canvas-1024x1024-64f": dict(name="canvas-1024x1024-64f", batch=1, heads=24, head_dim=128,
            frames=64, tokens_per_frame=4096, dtype="bf16", chunk=5,
            radius=1, rules=("vdn_solve",), c=0.5, text_tokens=256,
            alpha=(0.95, 1.0), seed=4),
}


def tiny_config(frames=17, radius=1, text_tokens=16, rule="vdn_solve",
                head_dim=16, tokens_per_frame=16, heads=1, dtype="f32",
                seed=100, alpha=(0.8, 1.0), chunk=5, batch=1, beta=(0.0, 1.0)):
    """Extra small cases: partial last chunk, text state on/off, radius 0;
    ``beta``: the range of the uniform beta draws (video and text tokens)."""
    return dict(name=f"tiny-F{frames}-r{radius}-T{text_tokens}-{rule}",
                batch=batch, heads=heads, head_dim=head_dim, frames=frames,
                tokens_per_frame=tokens_per_frame, dtype=dtype, chunk=chunk,
                radius=radius, rules=(rule,), c=0.5, text_tokens=text_tokens,
                alpha=alpha, seed=seed, beta=beta)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    """Host arrays of one workload. io tensors (q, k, v, gate, k_txt, v_txt)
    are float32 for ``dtype == 'f32'`` and uint16 bf16 bits for 'bf16'."""
    cfg: dict
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    gate: np.ndarray
    beta: np.ndarray
    alpha: np.ndarray
    conv_k: np.ndarray
    conv_v: np.ndarray
    rms_weight: np.ndarray
    k_txt: np.ndarray | None = None
    v_txt: np.ndarray | None = None
    beta_txt: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.cfg["frames"] * self.cfg["tokens_per_frame"]

    def f32(self, name: str, b=None, h=None) -> np.ndarray:
        """float32 view of an io tensor (whole, or one (b, h) slice)."""
        a = getattr(self, name)
        if b is not None:
            a = a[b, h]
        if self.cfg["dtype"] == "bf16" and a.dtype == np.uint16:
            return bf16_bits_to_f32(a)
        return np.asarray(a, dtype=np.float32)

    def f64(self, name: str, b=None, h=None) -> np.ndarray:
        return self.f32(name, b, h).astype(np.float64)


def _draw(seed, name, b, h, shape, kind, lo=0.0, hi=1.0, std=1.0):
    rng = np.random.default_rng([seed, TID[name], b, h])
    if kind == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return x
    x = rng.random(shape, dtype=np.float32)
    return (np.float32(lo) + np.float32(hi - lo) * x).astype(np.float32)


def make(cfg, *, beta_zero=False, alpha_one=False, identity_conv=False,
         random_rms_weight=False, workers=None) -> Inputs:
    """Generate the inputs of a workload.

    ``cfg`` is a key of :data:`WORKLOADS` or a workload dict. The switches replace
    a tensor by a constant for the special cases the tests use: beta = 0,
    alpha = 1, identity conv taps (1, 0, 0, 0); ``random_rms_weight`` draws
    the RMSNorm weight from U(0.5, 1.5) instead of ones.
    """
    if not isinstance(cfg, dict):
        cfg = WORKLOADS[cfg]
    cfg = dict(cfg)
    B, H, d = cfg["batch"], cfg["heads"], cfg["head_dim"]
    F, S = cfg["frames"], cfg["tokens_per_frame"]
    N = F * S
    T = cfg["text_tokens"]
    seed = cfg["seed"]
    bf16 = cfg["dtype"] == "bf16"
    io_dtype = np.uint16 if bf16 else np.float32
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))

    def io(x):
        return f32_to_bf16_bits(x) if bf16 else x

    q = np.empty((B, H, N, d), dtype=io_dtype)
    k = np.empty_like(q)
    v = np.empty_like(q)
    gate = np.empty_like(q)
    beta = np.empty((B, H, N), dtype=np.float32)
    alpha = np.empty((B, H, F, d), dtype=np.float32)
    if T > 0:
        k_txt = np.empty((B, H, T, d), dtype=io_dtype)
        v_txt = np.empty_like(k_txt)
        beta_txt = np.empty((B, H, T), dtype=np.float32)
    else:
        k_txt = v_txt = beta_txt = None

    def slice_job(bh):
        b, h = bh
        for name, arr in (("q", q), ("k", k), ("v", v), ("gate", gate)):
            arr[b, h] = io(_draw(seed, name, b, h, (N, d), "normal"))
        b_lo, b_hi = cfg.get("beta", (0.0, 1.0))
        beta[b, h] = 0.0 if beta_zero else _draw(seed, "beta", b, h, (N,), "uniform", b_lo, b_hi)
        a_lo, a_hi = cfg["alpha"]
        alpha[b, h] = 1.0 if alpha_one else _draw(seed, "alpha", b, h, (F, d),
                                                   "uniform", a_lo, a_hi)
        if T > 0:
            k_txt[b, h] = io(_draw(seed, "k_txt", b, h, (T, d), "normal"))
            v_txt[b, h] = io(_draw(seed, "v_txt", b, h, (T, d), "normal"))
            beta_txt[b, h] = _draw(seed, "beta_txt", b, h, (T,), "uniform", b_lo, b_hi)

    jobs = [(b, h) for b in range(B) for h in range(H)]
    if workers > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(slice_job, jobs))
    else:
        for j in jobs:
            slice_job(j)

    conv_k = np.empty((H, d, 4), dtype=np.float32)
    conv_v = np.empty_like(conv_k)
    for h in range(H):
        if identity_conv:
            conv_k[h] = 0.0
            conv_k[h, :, 0] = 1.0
            conv_v[h] = conv_k[h]
        else:
            conv_k[h] = _draw(seed, "conv_k", 0, h, (d, 4), "normal", std=0.5)
            conv_v[h] = _draw(seed, "conv_v", 0, h, (d, 4), "normal", std=0.5)
    rms_weight = (_draw(seed, "rms_weight", 0, 0, (d,), "uniform", 0.5, 1.5)
                  if random_rms_weight else np.ones(d, dtype=np.float32))
    return Inputs(cfg=cfg, q=q, k=k, v=v, gate=gate, beta=beta, alpha=alpha,
                  conv_k=conv_k, conv_v=conv_v, rms_weight=rms_weight,
                  k_txt=k_txt, v_txt=v_txt, beta_txt=beta_txt)


def grad_output(cfg) -> np.ndarray:
    """Upstream gradient dL/do ~ N(0, 1) of a workload, [B, H, N, d] in its
    I/O dtype (uint16 bf16 bits or float32), drawn like q."""
    if not isinstance(cfg, dict):
        cfg = WORKLOADS[cfg]
    B, H, d = cfg["batch"], cfg["heads"], cfg["head_dim"]
    N = cfg["frames"] * cfg["tokens_per_frame"]
    bf16 = cfg["dtype"] == "bf16"
    out = np.empty((B, H, N, d), dtype=np.uint16 if bf16 else np.float32)
    for b in range(B):
        for h in range(H):
            x = _draw(cfg["seed"], "d_out", b, h, (N, d), "normal")
            out[b, h] = f32_to_bf16_bits(x) if bf16 else x
    return out


def state_matrix(cfg) -> np.ndarray:
    """A text state S_text [B, H, d, d] float32 drawn directly, N(0, 1 / d)
    (the gradient tests feed the same matrix to both sides)."""
    if not isinstance(cfg, dict):
        cfg = WORKLOADS[cfg]
    B, H, d = cfg["batch"], cfg["heads"], cfg["head_dim"]
    out = np.empty((B, H, d, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h] = _draw(cfg["seed"], "state", b, h, (d, d), "normal", std=d ** -0.5)
    return out


def alpha_weights(cfg):
    """Synthetic weights of the per-frame forget-gate producer, per head:
    W [H, d, d] ~ N(0, 1/d), bias [H, d] ~ N(0, 1/4), a_log [H, d] =
    ln(0.05) + N(0, 1/25), float32 (with N(0, 1) keys the gates fall in
    about 0.90 .. 0.99, the range of the workloads' alpha draws)."""
    if not isinstance(cfg, dict):
        cfg = WORKLOADS[cfg]
    H, d, seed = cfg["heads"], cfg["head_dim"], cfg["seed"]
    w = np.stack([_draw(seed, "alpha_w", 0, h, (d, d), "normal", std=d ** -0.5)
                  for h in range(H)])
    b = np.stack([_draw(seed, "alpha_b", 0, h, (d,), "normal", std=0.5) for h in range(H)])
    a = np.stack([np.float32(np.log(0.05)) + _draw(seed, "alpha_a", 0, h, (d,), "normal",
                                                   std=0.2) for h in range(H)])
    return w.astype(np.float32), b.astype(np.float32), a.astype(np.float32)


def block_inputs(cfg):
    """Block input x [B, N, D] ~ N(0, 1) and the projections' synthetic
    weights W_qkv [3 D, D], W_o [D, D] ~ N(0, 1/D) (so q, k, v ~ N(0, 1) as in
    the attention workloads), D = heads * head_dim; bf16 bits (uint16).
    x of batch element b is drawn as slice (b, 0)."""
    if not isinstance(cfg, dict):
        cfg = WORKLOADS[cfg]
    B, H, d, seed = cfg["batch"], cfg["heads"], cfg["head_dim"], cfg["seed"]
    D = H * d
    N = cfg["frames"] * cfg["tokens_per_frame"]
    x = np.stack([f32_to_bf16_bits(_draw(seed, "x", b, 0, (N, D), "normal")) for b in range(B)])
    wq = f32_to_bf16_bits(_draw(seed, "w_qkv", 0, 0, (3 * D, D), "normal", std=D ** -0.5))
    wo = f32_to_bf16_bits(_draw(seed, "w_o", 0, 0, (D, D), "normal", std=D ** -0.5))
    return x, wq, wo
