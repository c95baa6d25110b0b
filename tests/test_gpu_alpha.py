"""GPU parity of the per-frame forget-gate producer (hwa_frame_alpha) with the
oracle's frame_alpha, through the C ABI, and of the forward fed with its
output.

alpha_f = exp(-exp(a) softplus(mean_f(k) W + b)) per (batch, head, frame,
channel), computed in fp32 from the (exact) dtype inputs: bar 1e-5 relative
Frobenius per (b, h) slice in both dtypes.
"""

import numpy as np
import pytest
import torch

import oracle
from hybrid_window_softmax_amd import hwa, inputs
from harness import (TOL, GpuCase, check_poisoned, oracle_text_state, out_f64, poisoned,
                     to_dev)

pytestmark = pytest.mark.gpu


def _check(cfg, guard=False):
    print(f"case alpha {cfg['name']} {cfg['dtype']} B{cfg['batch']} H{cfg['heads']} "
          f"d{cfg['head_dim']} F{cfg['frames']} S{cfg['tokens_per_frame']} guard={guard}",
          flush=True)
    inp = inputs.make(cfg)
    bf = cfg["dtype"] == "bf16"
    k = to_dev(inp.k, bf)
    w, b, a = (to_dev(x, False) for x in inputs.alpha_weights(cfg))
    B, H, F, d = cfg["batch"], cfg["heads"], cfg["frames"], cfg["head_dim"]
    out = flat = None
    if guard:
        out, flat = poisoned((B, H, F, d), torch.float32)
    got = hwa.frame_alpha(k, w, b, a, F, cfg["tokens_per_frame"], out=out)
    torch.cuda.synchronize()
    if guard:
        check_poisoned(got, flat, "alpha")
    got = got.cpu().numpy().astype(np.float64)
    wh, bh, ah = inputs.alpha_weights(cfg)
    worst = 0.0
    for bb in range(B):
        for h in range(H):
            ref = oracle.frame_alpha(inp.f64("k", bb, h), wh[h], bh[h], ah[h],
                                     cfg["tokens_per_frame"])
            worst = max(worst, oracle.rel_frobenius(got[bb, h], ref))
    print(f"  max rel Frobenius {worst:.3e}", flush=True)
    assert worst <= 1e-5, worst


@pytest.mark.parametrize("kw", [
    dict(),                                                        # fp32 d 16
    dict(head_dim=32, tokens_per_frame=37, frames=9, batch=2, heads=2),
    dict(head_dim=64, tokens_per_frame=256, frames=6, heads=3, dtype="bf16"),
    dict(head_dim=128, tokens_per_frame=1, frames=23, heads=2, dtype="bf16"),
    dict(head_dim=128, tokens_per_frame=100, frames=12, heads=2, dtype="bf16", batch=2),
])
def test_frame_alpha_small(kw):
    _check(inputs.tiny_config(text_tokens=0, seed=130, **kw))


def test_frame_alpha_full_size_guarded():
    # every head of the 132,600-token workload, the output poisoned and guarded
    _check(inputs.WORKLOADS["long-clip-832x480-85f"], guard=True)


@pytest.mark.parametrize("cfg", ["small-bf16-text",
                                 inputs.tiny_config(frames=17, text_tokens=16, head_dim=32,
                                                    tokens_per_frame=24, heads=2, seed=131)])
def test_forward_with_produced_alpha(cfg):
    # the gate producer feeding the forward: hwa_frame_alpha's alpha goes into
    # hybrid_attn_fwd; the oracle runs its own frame_alpha and the forward
    cfg = inputs.WORKLOADS[cfg] if isinstance(cfg, str) else cfg
    print(f"case forward with produced alpha {cfg['name']} {cfg['dtype']}", flush=True)
    inp = inputs.make(cfg)
    case = GpuCase(inp)
    t = case.t
    c = inp.cfg
    F, S = c["frames"], c["tokens_per_frame"]
    w, b, a = (to_dev(x, False) for x in inputs.alpha_weights(cfg))
    alpha = hwa.frame_alpha(t["k"], w, b, a, F, S)
    out, _ = hwa.hybrid_attn_fwd(t["q"], t["k"], t["v"], t["beta"], alpha, t["gate"],
                                 case.text_state, t["conv_k"], t["conv_v"], F, S, c["chunk"],
                                 c["radius"], "vdn_solve", c["c"], 0.5, 1e-6, t["rms_weight"])
    torch.cuda.synchronize()
    got = out_f64(out)
    wh, bh, ah = inputs.alpha_weights(cfg)
    worst = 0.0
    for bb in range(c["batch"]):
        for h in range(c["heads"]):
            al = oracle.frame_alpha(inp.f64("k", bb, h), wh[h], bh[h], ah[h], S)
            ref = oracle.hybrid_attn_head(
                inp.f64("q", bb, h), inp.f64("k", bb, h), inp.f64("v", bb, h), inp.beta[bb, h],
                al, inp.f64("gate", bb, h), oracle_text_state(inp, bb, h), inp.conv_k[h],
                inp.conv_v[h], inp.rms_weight, S, c["chunk"], c["radius"], "vdn_solve",
                c["c"], 0.5, 1e-6)[0]
            worst = max(worst, oracle.rel_frobenius(got[bb, h], ref))
    print(f"  out max rel Frobenius {worst:.3e}", flush=True)
    assert worst <= TOL[c["dtype"]], worst
