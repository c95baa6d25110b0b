"""GPU parity of the linear branch's backward (hwa_linear_bwd) with the fp64
oracle gradient (torch autograd of the branch, pinned by finite differences
of the numpy oracle), through the C ABI.

Every gradient is compared per (b, h) slice by relative Frobenius error;
the conv taps (per head) are compared summed over the batch and the RMSNorm
weight summed over batch and heads, as the library returns them. Without a
text state the library returns dL/dS_text at the zero state, which the
oracle gives for S_text = 0. Bar: 1e-5 (fp32) / 5e-3 (bf16: dq, dk, dv and
dgate are rounded to bf16, the fp32 outputs see the bf16 inputs only).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from hybrid_window_softmax_amd import hwa, inputs
from harness import (TOL, check_poisoned, check_workspace_guard, guarded_workspace,
                     poisoned, to_dev)

pytestmark = pytest.mark.gpu

PER_HEAD = ("q", "k", "v", "beta", "alpha", "gate", "text_state")


def _gpu_grads(inp, rule, st_host, g_host, guard=False):
    """hwa_linear_bwd's gradients as float64 host arrays. ``guard``: every
    output pre-filled with NaN inside NaN guard bands and the workspace inside
    0xA5 bands, checked after the call."""
    c = inp.cfg
    bf = c["dtype"] == "bf16"
    t = {n: to_dev(getattr(inp, n), bf) for n in
         ("q", "k", "v", "gate", "beta", "alpha", "conv_k", "conv_v", "rms_weight")}
    d_o = to_dev(g_host, bf)
    S_t = None if st_host is None else to_dev(st_host, False)
    grads = ws = None
    if guard:
        B, H, N, d = t["q"].shape
        F = c["frames"]
        io = t["q"].dtype
        shapes = dict(q=((B, H, N, d), io), k=((B, H, N, d), io), v=((B, H, N, d), io),
                      gate=((B, H, N, d), io), beta=((B, H, N), torch.float32),
                      alpha=((B, H, F, d), torch.float32),
                      text_state=((B, H, d, d), torch.float32),
                      conv_k=((H, d, 4), torch.float32), conv_v=((H, d, 4), torch.float32),
                      rms_weight=((d,), torch.float32))
        bufs = {n: poisoned(shp, dt) for n, (shp, dt) in shapes.items()}
        grads = {n: b[0] for n, b in bufs.items()}
        p = hwa.make_params(B, H, d, io)
        need = int(hwa.lib().hwa_linear_bwd_workspace_bytes(F, c["tokens_per_frame"],
                                                            c["chunk"], ctypes.byref(p)))
        ws, ws_flat = guarded_workspace(need)
    grads, _ = hwa.linear_bwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"], S_t,
                              t["conv_k"], t["conv_v"], d_o, c["frames"], c["tokens_per_frame"],
                              c["chunk"], c["radius"], rule, c["c"], 0.5, 1e-6, t["rms_weight"],
                              grads=grads, workspace=ws)
    torch.cuda.synchronize()
    if guard:
        for n, (view, flat) in bufs.items():
            check_poisoned(view, flat, f"{c['name']} d{n}")
        check_workspace_guard(ws_flat, need, f"{c['name']} linear backward")
    return {n: x.float().cpu().numpy().astype(np.float64) for n, x in grads.items()}


def _f64(inp, x):
    if inp.cfg["dtype"] == "bf16" and x.dtype == np.uint16:
        return inputs.bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, np.float64)


def check(inp, rule="vdn_solve", text=True):
    c = inp.cfg
    print(f"case {c['name']} {c['dtype']} B{c['batch']} H{c['heads']} d{c['head_dim']} "
          f"F{c['frames']} S{c['tokens_per_frame']} chunk {c['chunk']} r {c['radius']} "
          f"{rule} text {text}", flush=True)
    g_host = inputs.grad_output(c)
    st_host = inputs.state_matrix(c) if text else None
    got = _gpu_grads(inp, rule, st_host, g_host)
    B, H, d = c["batch"], c["heads"], c["head_dim"]
    worst = dict.fromkeys(PER_HEAD, 0.0)
    conv_k = np.zeros((H, d, 4))
    conv_v = np.zeros((H, d, 4))
    w = np.zeros(d)
    for b in range(B):
        for h in range(H):
            S_text = st_host[b, h] if text else np.zeros((d, d))
            ref = oracle.linear_branch_grad(
                inp.f64("q", b, h), inp.f64("k", b, h), inp.f64("v", b, h), inp.beta[b, h],
                inp.alpha[b, h], inp.f64("gate", b, h), S_text, inp.conv_k[h], inp.conv_v[h],
                inp.rms_weight, _f64(inp, g_host[b, h]), c["tokens_per_frame"], c["chunk"],
                c["radius"], rule, c["c"], 0.5, 1e-6)
            for n in PER_HEAD:
                r = ref["S_text" if n == "text_state" else n]
                worst[n] = max(worst[n], oracle.rel_frobenius(got[n][b, h], r))
            conv_k[h] += ref["conv_k"]
            conv_v[h] += ref["conv_v"]
            w += ref["w"]
    worst["conv_k"] = oracle.rel_frobenius(got["conv_k"], conv_k)
    worst["conv_v"] = oracle.rel_frobenius(got["conv_v"], conv_v)
    worst["rms_weight"] = oracle.rel_frobenius(got["rms_weight"], w)
    print("  rel err " + " ".join(f"d{n} {e:.2e}" for n, e in worst.items()), flush=True)
    tol = TOL[c["dtype"]]
    assert max(worst.values()) <= tol, worst


def test_tiny_fp32_160tok():
    check(inputs.make("tiny-f32"))


@pytest.mark.parametrize("kw,rule,text", [
    (dict(frames=17, head_dim=32, tokens_per_frame=37), "vdn_scaled", True),   # partial chunk
    (dict(frames=12, head_dim=64, tokens_per_frame=20, batch=2, heads=2, radius=0),
     "vdn_solve", False),
    (dict(frames=14, head_dim=128, tokens_per_frame=24, chunk=3), "vdn_solve", True),
    (dict(frames=6, head_dim=16, tokens_per_frame=3, chunk=1), "vdn_scaled", True),  # S < taps
])
def test_small_fp32(kw, rule, text):
    check(inputs.make(inputs.tiny_config(text_tokens=0, seed=400, **kw),
                      random_rms_weight=True), rule, text)


def test_small_bf16_5120tok():
    check(inputs.make("small-bf16-text", random_rms_weight=True))


@pytest.mark.parametrize("kw,rule", [
    (dict(frames=11, head_dim=128, tokens_per_frame=45, heads=2), "vdn_scaled"),
    (dict(frames=1, head_dim=64, tokens_per_frame=1), "vdn_solve"),             # one token
])
def test_bf16_shapes(kw, rule):
    check(inputs.make(inputs.tiny_config(text_tokens=0, dtype="bf16", seed=401, **kw)), rule)


def test_repeat_bit_exact():
    # no atomics: every output element is one fixed sum
    inp = inputs.make("small-bf16-text")
    c = inp.cfg
    print("case small-bf16-text: two calls agree bit for bit", flush=True)
    g_host = inputs.grad_output(c)
    st = inputs.state_matrix(c)
    a = _gpu_grads(inp, "vdn_solve", st, g_host)
    b = _gpu_grads(inp, "vdn_solve", st, g_host)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("kw,text", [
    # the far field on both sides of every window (chunks of 2, radius 0)
    (dict(frames=12, head_dim=32, tokens_per_frame=8, chunk=2, radius=0), True),
    (dict(frames=9, head_dim=64, tokens_per_frame=20, batch=2, heads=2), False),
    (dict(frames=14, head_dim=128, tokens_per_frame=24, chunk=3), True),
])
def test_sana_scaled_fp32(kw, text):
    # sana_scaled: S_f = (S_{f-1} D_f)(I - c^2 A_f) + c B_f; at these sizes the
    # states stay well inside fp32's range (the backward carries no exponents)
    check(inputs.make(inputs.tiny_config(text_tokens=0, seed=403, **kw),
                      random_rms_weight=True), "sana_scaled", text)


def test_sana_scaled_bf16():
    check(inputs.make(inputs.tiny_config(frames=11, head_dim=128, tokens_per_frame=45, heads=2,
                                         text_tokens=0, dtype="bf16", seed=404)),
          "sana_scaled")


def test_long_clip_132600tok_one_head():
    # the full workload (24 heads, 85 frames of 1560 tokens) on the GPU; every
    # gradient of head 5 against the oracle (the batch is 1, so that head's
    # conv-tap gradients are the library's; the RMSNorm weight's sums over
    # all heads and is covered by the smaller cases)
    name = "long-clip-832x480-85f"
    inp = inputs.make(name)
    c = inp.cfg
    h = 5
    print(f"case {name}: all heads on the GPU (outputs poisoned and guarded), head {h} "
          "against the oracle", flush=True)
    g_host = inputs.grad_output(c)
    st_host = inputs.state_matrix(c)
    got = _gpu_grads(inp, "vdn_solve", st_host, g_host, guard=True)
    ref = oracle.linear_branch_grad(
        inp.f64("q", 0, h), inp.f64("k", 0, h), inp.f64("v", 0, h), inp.beta[0, h],
        inp.alpha[0, h], inp.f64("gate", 0, h), st_host[0, h], inp.conv_k[h], inp.conv_v[h],
        inp.rms_weight, _f64(inp, g_host[0, h]), c["tokens_per_frame"], c["chunk"],
        c["radius"], "vdn_solve", c["c"], 0.5, 1e-6)
    errs = {n: oracle.rel_frobenius(got[n][0, h], ref["S_text" if n == "text_state" else n])
            for n in PER_HEAD}
    errs["conv_k"] = oracle.rel_frobenius(got["conv_k"][h], ref["conv_k"])
    errs["conv_v"] = oracle.rel_frobenius(got["conv_v"][h], ref["conv_v"])
    print("  rel err " + " ".join(f"d{n} {e:.2e}" for n, e in errs.items()), flush=True)
    assert max(errs.values()) <= TOL["bf16"], errs


@pytest.mark.parametrize("cfg,rule", [
    ("small-bf16-text", "vdn_solve"),
    (inputs.tiny_config(frames=17, head_dim=32, tokens_per_frame=37, text_tokens=0, seed=402),
     "vdn_scaled"),
    (inputs.tiny_config(frames=10, head_dim=64, tokens_per_frame=16, text_tokens=0, seed=405),
     "sana_scaled"),
])
def test_hybrid_autograd(cfg, rule):
    # hwa.hybrid_attention through torch autograd: out.backward(g) runs
    # hwa_softmax_bwd, then hwa_linear_bwd accumulating into dq, dk, dv; every
    # gradient against the oracle (softmax-branch gradient + linear-branch
    # gradient for q, k, v)
    inp = inputs.make(cfg, random_rms_weight=True)
    c = inp.cfg
    bf = c["dtype"] == "bf16"
    print(f"case {c['name']} {c['dtype']}: hybrid attention autograd, {rule}", flush=True)
    t = {n: to_dev(getattr(inp, n), bf).requires_grad_() for n in
         ("q", "k", "v", "gate", "beta", "alpha", "conv_k", "conv_v", "rms_weight")}
    st_host = inputs.state_matrix(c)
    text = to_dev(st_host, False).requires_grad_()
    g_host = inputs.grad_output(c)
    F, S, ch, r = c["frames"], c["tokens_per_frame"], c["chunk"], c["radius"]
    out = hwa.hybrid_attention(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"], text,
                               t["conv_k"], t["conv_v"], F, S, ch, r, rule, c["c"], 0.5, 1e-6,
                               t["rms_weight"])
    out.backward(to_dev(g_host, bf))
    torch.cuda.synchronize()
    got = {n: x.grad.float().cpu().numpy().astype(np.float64) for n, x in t.items()}
    got["text_state"] = text.grad.cpu().numpy().astype(np.float64)
    lo, hi = oracle.window_bounds(F, ch, r)
    B, H, d = c["batch"], c["heads"], c["head_dim"]
    worst = dict.fromkeys(PER_HEAD, 0.0)
    conv_k, conv_v, w = np.zeros((H, d, 4)), np.zeros((H, d, 4)), np.zeros(d)
    for b in range(B):
        for h in range(H):
            q, k, v = (inp.f64(n, b, h) for n in ("q", "k", "v"))
            g = _f64(inp, g_host[b, h])
            ref = oracle.linear_branch_grad(
                q, k, v, inp.beta[b, h], inp.alpha[b, h], inp.f64("gate", b, h), st_host[b, h],
                inp.conv_k[h], inp.conv_v[h], inp.rms_weight, g, S, ch, r, rule, c["c"], 0.5,
                1e-6)
            sq, sk, sv = oracle.softmax_branch_grad(q, k, v, g, S, lo, hi)
            ref["q"], ref["k"], ref["v"] = ref["q"] + sq, ref["k"] + sk, ref["v"] + sv
            for n in PER_HEAD:
                rr = ref["S_text" if n == "text_state" else n]
                worst[n] = max(worst[n], oracle.rel_frobenius(got[n][b, h], rr))
            conv_k[h] += ref["conv_k"]
            conv_v[h] += ref["conv_v"]
            w += ref["w"]
    worst["conv_k"] = oracle.rel_frobenius(got["conv_k"], conv_k)
    worst["conv_v"] = oracle.rel_frobenius(got["conv_v"], conv_v)
    worst["rms_weight"] = oracle.rel_frobenius(got["rms_weight"], w)
    print("  rel err " + " ".join(f"d{n} {e:.2e}" for n, e in worst.items()), flush=True)
    assert max(worst.values()) <= TOL[c["dtype"]], worst


@pytest.mark.parametrize("name,h", [("clip-832x480-31f", 23), ("canvas-1024x1024-64f", 11)])
def test_full_size_one_head(name, h):
    # the other full-size workloads: every head on the GPU, one head against
    # the oracle in full (batch 1: that head's conv-tap gradients are the
    # library's)
    inp = inputs.make(name)
    c = inp.cfg
    print(f"case {name}: all heads on the GPU (outputs poisoned and guarded), head {h} "
          "against the oracle", flush=True)
    g_host = inputs.grad_output(c)
    st_host = inputs.state_matrix(c)
    got = _gpu_grads(inp, "vdn_solve", st_host, g_host, guard=True)
    ref = oracle.linear_branch_grad(
        inp.f64("q", 0, h), inp.f64("k", 0, h), inp.f64("v", 0, h), inp.beta[0, h],
        inp.alpha[0, h], inp.f64("gate", 0, h), st_host[0, h], inp.conv_k[h], inp.conv_v[h],
        inp.rms_weight, _f64(inp, g_host[0, h]), c["tokens_per_frame"], c["chunk"],
        c["radius"], "vdn_solve", c["c"], 0.5, 1e-6)
    errs = {n: oracle.rel_frobenius(got[n][0, h], ref["S_text" if n == "text_state" else n])
            for n in PER_HEAD}
    errs["conv_k"] = oracle.rel_frobenius(got["conv_k"][h], ref["conv_k"])
    errs["conv_v"] = oracle.rel_frobenius(got["conv_v"][h], ref["conv_v"])
    print("  rel err " + " ".join(f"d{n} {e:.2e}" for n, e in errs.items()), flush=True)
    assert max(errs.values()) <= TOL["bf16"], errs


@pytest.mark.parametrize("dtype,d", [("f32", 32), ("bf16", 128)])
def test_negative_beta(dtype, d):
    # beta ~ U(-0.5, 1): negative writes in the statistics (on bf16 calls the
    # frames that hold one are recomputed by the fp32 statistics kernel); with
    # and without a text state
    for text in (True, False):
        check(inputs.make(inputs.tiny_config(frames=12, text_tokens=0, head_dim=d,
                                             tokens_per_frame=40, dtype=dtype, heads=2,
                                             seed=403, beta=(-0.5, 1.0))), "vdn_solve", text)
