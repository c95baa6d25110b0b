"""Shared helpers of the parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same seeded inputs, and compare them."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from hybrid_window_softmax_amd import hwa, inputs

TOL = {"f32": 1e-5, "bf16": 5e-3}


def to_dev(a: np.ndarray, bf16: bool, dev="cuda"):
    if a is None:
        return None
    if bf16 and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


class GpuCase:
    """Device copies of one workload and calls of the library on them."""

    def __init__(self, inp: inputs.Inputs, dev="cuda"):
        self.inp = inp
        cfg = inp.cfg
        self.cfg = cfg
        bf = cfg["dtype"] == "bf16"
        self.bf16 = bf
        self.t = {n: to_dev(getattr(inp, n), bf, dev)
                  for n in ("q", "k", "v", "gate", "beta", "alpha", "conv_k", "conv_v",
                            "rms_weight", "k_txt", "v_txt", "beta_txt")}
        self.text_state = None
        if inp.k_txt is not None:
            self.text_state = hwa.text_state(self.t["k_txt"], self.t["v_txt"],
                                             self.t["beta_txt"])

    def run(self, rule="vdn_solve", flags=0, text=True, out=None, workspace=None, rope=None):
        """rope: optional (q_rope, k_rope) host arrays for the softmax branch."""
        c = self.cfg
        t = self.t
        qr = kr = None
        if rope is not None:
            qr, kr = (to_dev(a, self.bf16) for a in rope)
        return hwa.hybrid_attn_fwd(
            t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"],
            self.text_state if text else None, t["conv_k"], t["conv_v"],
            c["frames"], c["tokens_per_frame"], c["chunk"], c["radius"], rule, c["c"],
            0.5, 1e-6, t["rms_weight"], q_rope=qr, k_rope=kr, flags=flags, out=out,
            workspace=workspace)

    def layout(self):
        c = self.cfg
        p = hwa.make_params(c["batch"], c["heads"], c["head_dim"],
                            torch.bfloat16 if self.bf16 else torch.float32)
        return hwa.workspace_layout(c["frames"], c["tokens_per_frame"], c["chunk"], p)


def ws_view(ws: torch.Tensor, offset: int, shape, dtype=torch.float32):
    n = int(np.prod(shape))
    es = torch.tensor([], dtype=dtype).element_size()
    return ws[offset:offset + n * es].view(dtype).view(*shape)


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def oracle_text_state(inp, b, h):
    if inp.k_txt is None:
        return None
    return oracle.text_state(inp.f64("k_txt", b, h), inp.f64("v_txt", b, h),
                             inp.beta_txt[b, h].astype(np.float64))


def oracle_head(inp, b, h, rule="vdn_solve", text=True, keep=False, rope=None):
    """(out, o_sm, y, intermediates) of one (b, h) in fp64; rope: optional
    (q_rope, k_rope) fp64 [N, d] slices for the softmax branch."""
    c = inp.cfg
    st = oracle_text_state(inp, b, h) if text else None
    qr, kr = rope if rope is not None else (None, None)
    return oracle.hybrid_attn_head(
        inp.f64("q", b, h), inp.f64("k", b, h), inp.f64("v", b, h),
        inp.beta[b, h].astype(np.float64), inp.alpha[b, h].astype(np.float64),
        inp.f64("gate", b, h), st, inp.conv_k[h], inp.conv_v[h], inp.rms_weight,
        c["tokens_per_frame"], c["chunk"], c["radius"], rule, c["c"], 0.5, 1e-6,
        q_rope=qr, k_rope=kr, keep=keep)


def oracle_linear_head(inp, b, h, rule="vdn_solve", text=True, keep=False):
    c = inp.cfg
    st = oracle_text_state(inp, b, h) if text else None
    return oracle.linear_branch(
        inp.f64("q", b, h), inp.f64("k", b, h), inp.f64("v", b, h),
        inp.beta[b, h].astype(np.float64), inp.alpha[b, h].astype(np.float64),
        inp.f64("gate", b, h), st, inp.conv_k[h], inp.conv_v[h], inp.rms_weight,
        c["tokens_per_frame"], c["chunk"], c["radius"], rule, c["c"], 0.5, 1e-6,
        keep=keep)


def sample_rows(cfg, n_random=48, seed=0):
    """Query rows that cover chunk starts/ends, 128-row tile edges, the last
    row and random rows."""
    F, S, ch = cfg["frames"], cfg["tokens_per_frame"], cfg["chunk"]
    N = F * S
    rows = set()
    for c0 in range(0, F, ch):
        a, e = c0 * S, min(F, c0 + ch) * S
        rows.update({a, a + 1, e - 1, e - 2})
        for x in (127, 128, 255, 256):
            if a + x < e:
                rows.add(a + x)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, N, n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N), dtype=np.int64)


def oracle_softmax_rows(inp, b, h, rows):
    c = inp.cfg
    lo, hi = oracle.window_bounds(c["frames"], c["chunk"], c["radius"])
    return oracle.softmax_rows(inp.f32("q", b, h), inp.f32("k", b, h), inp.f32("v", b, h),
                               c["tokens_per_frame"], lo, hi, rows)


# ---------------------------------------------------------------- guard bands
GUARD = 4096  # elements (bytes for the workspace) of poison around a buffer


def poisoned(shape, dtype, dev="cuda", guard=GUARD):
    """An output buffer pre-filled with NaN and surrounded by `guard` NaN
    elements on each side. Returns (view, flat): the view is what the library
    writes, flat holds the guard bands for :func:`check_poisoned`."""
    n = int(np.prod(shape))
    flat = torch.full((n + 2 * guard,), float("nan"), dtype=dtype, device=dev)
    return flat[guard:guard + n].view(*shape), flat


def check_poisoned(view, flat, name, guard=GUARD):
    """Every element the call should write is finite, and both guard bands
    still hold the exact NaN bit pattern they were filled with."""
    n = view.numel()
    bits = torch.int16 if flat.element_size() == 2 else torch.int32
    pat = torch.full((1,), float("nan"), dtype=flat.dtype, device=flat.device).view(bits)
    fb = flat.view(bits)
    assert torch.equal(fb[:guard], pat.expand(guard)), f"{name}: guard before the buffer written"
    assert torch.equal(fb[guard + n:], pat.expand(guard)), f"{name}: guard after the buffer written"
    bad = (~torch.isfinite(view.float())).sum().item()
    assert bad == 0, f"{name}: {bad} elements left unwritten (NaN) or non-finite"


def guarded_workspace(nbytes, dev="cuda", guard=GUARD):
    """A workspace of exactly `nbytes` (256-byte aligned) with `guard` bytes of
    0xA5 before and after it. Returns (view, flat)."""
    flat = torch.full((nbytes + 2 * guard,), 0xA5, dtype=torch.uint8, device=dev)
    return flat[guard:guard + nbytes], flat


def check_workspace_guard(flat, nbytes, name, guard=GUARD):
    assert bool((flat[:guard] == 0xA5).all()), f"{name}: bytes before the workspace written"
    assert bool((flat[guard + nbytes:] == 0xA5).all()), f"{name}: bytes after the workspace written"
