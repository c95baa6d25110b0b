"""GPU parity of the windowed-softmax backward (hwa_softmax_bwd) with the fp64
oracle's gradient, through the C ABI.

The forward runs with HWA_FLAG_SOFTMAX_ONLY and hands its log-sum-exp to the
backward; the oracle differentiates the same (dtype-rounded) q, k, v with the
same upstream gradient. Bar: max relative Frobenius error over (b, h) of dq,
dk and dv <= 1e-5 (fp32) / 5e-3 (bf16: a CPU emulation of the kernels'
rounding points -- bf16 p and ds operands, fp32 accumulation, bf16 outputs --
predicts 2.3e-3 to 2.4e-3 at d = 64 and 128).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from hybrid_window_softmax_amd import hwa, inputs
from harness import (TOL, GpuCase, check_poisoned, check_workspace_guard,
                     guarded_workspace, poisoned, sample_rows, to_dev)

pytestmark = pytest.mark.gpu

LSE_TOL = {"f32": 2e-5, "bf16": 4e-3}  # absolute, natural-log units


def _run(inp, g_host, guard=False):
    """Forward (softmax only, for the lse) then hwa_softmax_bwd. ``guard``:
    dq, dk, dv pre-filled with NaN inside NaN guard bands and the workspace
    inside 0xA5 bands; checked after the call (every element written, no
    byte past a buffer)."""
    c = inp.cfg
    bf = c["dtype"] == "bf16"
    q, k, v = (to_dev(getattr(inp, n), bf) for n in ("q", "k", "v"))
    g = to_dev(g_host, bf)
    B, H, N, d = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    F, S = c["frames"], c["tokens_per_frame"]
    o, _ = hwa.hybrid_attn_fwd(q, k, v, None, None, None, None, None, None, F, S, c["chunk"],
                               c["radius"], flags=hwa.FLAG_SOFTMAX_ONLY, softmax_lse=lse)
    if guard:
        bufs = [poisoned((B, H, N, d), q.dtype) for _ in range(3)]
        p = hwa.make_params(B, H, d, q.dtype)
        need = int(hwa.lib().hwa_softmax_bwd_workspace_bytes(F, S, c["chunk"], ctypes.byref(p)))
        ws, ws_flat = guarded_workspace(need)
        dq, dk, dv, _ = hwa.softmax_bwd(q, k, v, o, lse, g, F, S, c["chunk"], c["radius"],
                                        dq=bufs[0][0], dk=bufs[1][0], dv=bufs[2][0], workspace=ws)
        torch.cuda.synchronize()
        for (view, flat), nm in zip(bufs, ("dq", "dk", "dv")):
            check_poisoned(view, flat, f"{c['name']} {nm}")
        check_workspace_guard(ws_flat, need, f"{c['name']} softmax backward")
    else:
        dq, dk, dv, _ = hwa.softmax_bwd(q, k, v, o, lse, g, F, S, c["chunk"], c["radius"])
    torch.cuda.synchronize()
    # float32 host copies (exact for both dtypes); heads are widened one at a time
    return (lse.cpu().numpy().astype(np.float64),
            *(t.float().cpu().numpy() for t in (dq, dk, dv)))


def _g64(inp, g_host, b, h):
    x = g_host[b, h]
    if inp.cfg["dtype"] == "bf16":
        return inputs.bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def _rel(x, r, scale):
    """Relative Frobenius error; where the exact gradient is zero (one key in
    the window: p = 1, so ds = g.v - g.o vanishes), the kernel returns the
    fp32 rounding residue of that difference, which is held to the tolerance
    relative to the size of the terms it cancels (``scale``)."""
    nr = np.linalg.norm(r)
    if nr == 0.0:
        return np.linalg.norm(x) / scale
    return oracle.rel_frobenius(x, r)


def _check_full(inp):
    c = inp.cfg
    print(f"case {c['name']}: B{c['batch']} H{c['heads']} d{c['head_dim']} "
          f"F{c['frames']} S{c['tokens_per_frame']} chunk {c['chunk']} r {c['radius']}",
          flush=True)
    g_host = inputs.grad_output(c)
    lse, dq, dk, dv = _run(inp, g_host)
    lo, hi = oracle.window_bounds(c["frames"], c["chunk"], c["radius"])
    S = c["tokens_per_frame"]
    tol = TOL[c["dtype"]]
    worst = [0.0, 0.0, 0.0]
    for b in range(c["batch"]):
        for h in range(c["heads"]):
            q, k, v = (inp.f64(n, b, h) for n in ("q", "k", "v"))
            g = _g64(inp, g_host, b, h)
            rq, rk, rv = oracle.softmax_branch_grad(q, k, v, g, S, lo, hi)
            rl = oracle.softmax_lse(q, k, S, lo, hi)
            assert np.abs(lse[b, h] - rl).max() <= LSE_TOL[c["dtype"]], (b, h)
            # |ds| <= |g| |v| per pair; dq, dk carry one more factor |k| or |q| / sqrt(d)
            d = q.shape[1]
            scale = (np.linalg.norm(g) * np.abs(v).max() * np.sqrt(d)
                     * max(np.abs(k).max(), np.abs(q).max()))
            for i, (x, r) in enumerate(((dq[b, h], rq), (dk[b, h], rk), (dv[b, h], rv))):
                worst[i] = max(worst[i], _rel(x.astype(np.float64), r, scale))
    print(f"  rel err dq {worst[0]:.2e} dk {worst[1]:.2e} dv {worst[2]:.2e}", flush=True)
    assert max(worst) <= tol, worst


def test_tiny_fp32_160tok():
    _check_full(inputs.make("tiny-f32"))


@pytest.mark.parametrize("kw", [
    dict(frames=17, head_dim=32, tokens_per_frame=16),            # partial last chunk
    dict(frames=12, radius=0, head_dim=64, tokens_per_frame=20),   # block-diagonal
    dict(frames=12, chunk=3, head_dim=128, tokens_per_frame=9, heads=2),
    dict(frames=7, radius=3, head_dim=16, tokens_per_frame=37, batch=2),  # one window
])
def test_small_fp32(kw):
    _check_full(inputs.make(inputs.tiny_config(text_tokens=0, seed=300, **kw)))


def test_small_bf16_5120tok():
    _check_full(inputs.make("small-bf16-text"))


@pytest.mark.parametrize("kw", [
    dict(frames=12, tokens_per_frame=100, head_dim=128, heads=2),              # ragged tiles
    dict(frames=23, tokens_per_frame=33, head_dim=128, chunk=3, radius=2, batch=2),
    dict(frames=9, tokens_per_frame=70, head_dim=64, radius=0, heads=3),
    dict(frames=1, tokens_per_frame=1, head_dim=128),                          # one token
    dict(frames=5, tokens_per_frame=1, head_dim=64, chunk=1),                  # chunk of one
    dict(frames=6, tokens_per_frame=300, head_dim=128, radius=4),              # window = all
])
def test_bf16_shapes(kw):
    _check_full(inputs.make(inputs.tiny_config(text_tokens=0, dtype="bf16", seed=301, **kw)))


def _key_rows(cfg, chunks, seed):
    F, S, ch = cfg["frames"], cfg["tokens_per_frame"], cfg["chunk"]
    rows = set()
    rng = np.random.default_rng(seed)
    for c in chunks:
        a, e = c * ch * S, min(F, (c + 1) * ch) * S
        rows.update({a, a + 1, a + 127, a + 128, e - 1, e - 2})
        rows.update(rng.integers(a, e, 12).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _check_sampled(name, heads, chunks=3):
    inp = inputs.make(name)
    c = inp.cfg
    print(f"case {name}: sampled rows of heads {heads} + sums over every head, outputs "
          "poisoned and guarded", flush=True)
    g_host = inputs.grad_output(c)
    lse, dq, dk, dv = _run(inp, g_host, guard=True)
    F, S = c["frames"], c["tokens_per_frame"]
    nch = (F + c["chunk"] - 1) // c["chunk"]
    lo, hi = oracle.window_bounds(F, c["chunk"], c["radius"])
    tol = TOL["bf16"]
    # every head: sum_m dv_m = sum_n g_n (rows of p sum to one) and
    # sum_m dk_m = 0 (a shift of every key leaves every softmax unchanged),
    # up to the rounding of the outputs (about 2.4e-3 of ||dk||_F)
    for b in range(c["batch"]):
        for h in range(c["heads"]):
            gs = _g64(inp, g_host, b, h).sum(axis=0)
            dvs = dv[b, h].astype(np.float64).sum(axis=0)
            dkh = dk[b, h].astype(np.float64)
            assert np.linalg.norm(dvs - gs) <= 1e-2 * np.linalg.norm(gs), (b, h)
            assert np.linalg.norm(dkh.sum(axis=0)) <= 1e-2 * np.linalg.norm(dkh), (b, h)
    qrows = sample_rows(c, n_random=32, seed=5)
    krows = _key_rows(c, sorted({0, nch // 2, nch - 1})[:chunks], seed=6)
    for (b, h) in heads:
        q, k, v = (inp.f64(n, b, h) for n in ("q", "k", "v"))
        g = _g64(inp, g_host, b, h)
        rq, rk, rv = oracle.softmax_grad_rows(q, k, v, g, S, lo, hi, qrows, krows)
        errs = (oracle.rel_frobenius(dq[b, h][qrows].astype(np.float64), rq),
                oracle.rel_frobenius(dk[b, h][krows].astype(np.float64), rk),
                oracle.rel_frobenius(dv[b, h][krows].astype(np.float64), rv))
        print(f"  head {(b, h)}: rel err dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}",
              flush=True)
        assert max(errs) <= tol, errs


def test_clip_48360tok_sampled():
    _check_sampled("clip-832x480-31f", [(0, 0), (0, 23)])


def test_long_clip_132600tok_sampled():
    _check_sampled("long-clip-832x480-85f", [(0, 5)])


def test_canvas_262144tok_sampled():
    _check_sampled("canvas-1024x1024-64f", [(0, 17)], chunks=2)


@pytest.mark.parametrize("name", ["tiny-f32", "small-bf16-text"])
def test_forward_softmax_outputs(name):
    # softmax_out and softmax_lse of a call that runs both branches (bf16:
    # the fused readout path) equal the softmax-only call's out and lse bit
    # for bit, and asking for them leaves out unchanged
    inp = inputs.make(name)
    gc = GpuCase(inp)
    print(f"case {name}: forward softmax outputs", flush=True)
    t = gc.t
    B, H, N, d = t["q"].shape
    so = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    lse1 = torch.empty_like(lse)
    c = inp.cfg
    ref, _ = gc.run()
    args = (t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"], gc.text_state,
            t["conv_k"], t["conv_v"], c["frames"], c["tokens_per_frame"], c["chunk"],
            c["radius"], "vdn_solve", c["c"], 0.5, 1e-6, t["rms_weight"])
    out, _ = hwa.hybrid_attn_fwd(*args, softmax_lse=lse, softmax_out=so)
    sm, _ = hwa.hybrid_attn_fwd(*args, flags=hwa.FLAG_SOFTMAX_ONLY, softmax_lse=lse1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(so, sm)
    assert torch.equal(lse, lse1)
    assert bool(torch.isfinite(lse).all())


def test_autograd_function_small_bf16():
    # hwa.windowed_softmax_attention through torch autograd: o_sm.backward(g)
    # gives the library's dq, dk, dv, checked against the oracle gradient
    inp = inputs.make("small-bf16-text")
    c = inp.cfg
    print("case small-bf16-text: autograd function", flush=True)
    q, k, v = (to_dev(getattr(inp, n), True).requires_grad_() for n in ("q", "k", "v"))
    g_host = inputs.grad_output(c)
    o = hwa.windowed_softmax_attention(q, k, v, c["frames"], c["tokens_per_frame"], c["chunk"],
                                       c["radius"])
    o.backward(to_dev(g_host, True))
    torch.cuda.synchronize()
    lo, hi = oracle.window_bounds(c["frames"], c["chunk"], c["radius"])
    S = c["tokens_per_frame"]
    worst = 0.0
    for h in (0, c["heads"] - 1):
        ref = oracle.softmax_branch_grad(inp.f64("q", 0, h), inp.f64("k", 0, h),
                                         inp.f64("v", 0, h), _g64(inp, g_host, 0, h), S, lo, hi)
        for t, r in zip((q, k, v), ref):
            worst = max(worst, oracle.rel_frobenius(
                t.grad[0, h].float().cpu().numpy().astype(np.float64), r))
    print(f"  rel err {worst:.2e}", flush=True)
    assert worst <= TOL["bf16"]
