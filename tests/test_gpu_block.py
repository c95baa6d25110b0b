"""GPU parity of the attention block (hwa_block_fwd: QKV projection with the
3D RoPE fused into its epilogue, the hybrid attention, output projection)
with the fp64 block oracle (oracle.block_fwd), through the C ABI.

Bars: the block output y against the fp64 definition within the bf16 bar
5e-3 (a CPU emulation of the rounding points -- q, k, v, their rotations and
the attention output stored as bf16, y rounded -- puts that error at about
3.6e-3); against the oracle with those same rounding points within 3e-3 (what
is left is the attention's own error, about 1.7e-3 on its bf16 output, carried
through W_o, and y's rounding); the projection's q, k, v and rotations
(workspace) per head within 5e-3 (their bf16 rounding, 1.7e-3).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from hybrid_window_softmax_amd import hwa, inputs
from harness import (check_poisoned, check_workspace_guard, guarded_workspace,
                     oracle_text_state, poisoned, to_dev)

pytestmark = pytest.mark.gpu


def _bf(a):
    return inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(
        np.float64)


def _check(cfg, grid_w, rule="vdn_solve", guard=False, check_qkv=False):
    print(f"case block {cfg['name']} B{cfg['batch']} H{cfg['heads']} d{cfg['head_dim']} "
          f"F{cfg['frames']} S{cfg['tokens_per_frame']} grid_w {grid_w} {rule} guard={guard}",
          flush=True)
    inp = inputs.make(cfg)
    xb, wqb, wob = inputs.block_inputs(cfg)
    B, H, d = cfg["batch"], cfg["heads"], cfg["head_dim"]
    F, S = cfg["frames"], cfg["tokens_per_frame"]
    N, D = F * S, H * d
    dev = "cuda"
    t = {n: to_dev(getattr(inp, n), True) for n in
         ("beta", "alpha", "gate", "conv_k", "conv_v", "rms_weight", "k_txt", "v_txt",
          "beta_txt")}
    text = None
    if inp.k_txt is not None:
        text = hwa.text_state(t["k_txt"], t["v_txt"], t["beta_txt"])
    x, wq, wo = (to_dev(a, True) for a in (xb, wqb, wob))
    y = ws = None
    if guard:
        y, y_flat = poisoned((B, N, D), torch.bfloat16)
        p = hwa.make_params(B, H, d, torch.bfloat16)
        need = int(hwa.lib().hwa_block_workspace_bytes(F, S, cfg["chunk"], ctypes.byref(p)))
        ws, ws_flat = guarded_workspace(need)
    y, ws = hwa.block_fwd(x, wq, wo, t["beta"], t["alpha"], t["gate"], text, t["conv_k"],
                          t["conv_v"], H, F, S, grid_w, 10000.0, cfg["chunk"], cfg["radius"], rule,
                          cfg["c"], 0.5, 1e-6, t["rms_weight"], y=y, workspace=ws)
    torch.cuda.synchronize()
    if guard:
        check_poisoned(y, y_flat, "block y")
        check_workspace_guard(ws_flat, need, "block")
    got = y.float().cpu().numpy().astype(np.float64)
    wq64 = inputs.bf16_bits_to_f32(wqb).astype(np.float64)
    wo64 = inputs.bf16_bits_to_f32(wob).astype(np.float64)
    worst = {"y": 0.0, "y_rounded": 0.0, "qkv": 0.0}
    io = B * H * N * d * 2
    r = -(-io // 256) * 256
    for b in range(B):
        x64 = inputs.bf16_bits_to_f32(xb[b]).astype(np.float64)
        st = None
        if inp.k_txt is not None:
            st = np.stack([oracle_text_state(inp, b, h) for h in range(H)])
        gate = np.stack([inp.f64("gate", b, h) for h in range(H)])
        args = (x64, wq64, wo64, inp.beta[b].astype(np.float64), inp.alpha[b].astype(np.float64),
                gate, st, inp.conv_k, inp.conv_v, inp.rms_weight, H, S, grid_w, 10000.0,
                cfg["chunk"], cfg["radius"], rule, cfg["c"], 0.5, 1e-6)
        ref = oracle.block_fwd(*args)
        ref_r = _bf(oracle.block_fwd(*args, round_to=_bf))
        worst["y"] = max(worst["y"], oracle.rel_frobenius(got[b], ref))
        worst["y_rounded"] = max(worst["y_rounded"], oracle.rel_frobenius(got[b], ref_r))
        if check_qkv:
            # the projection's outputs in the workspace: q, k, v, q_rope, k_rope
            qkv = x64 @ wq64.T
            for which in range(5):
                view = ws[which * r:which * r + io].view(torch.bfloat16).view(B, H, N, d)
                g = view[b].float().cpu().numpy().astype(np.float64)
                for h in range(H):
                    src = qkv[:, (which % 3) * D + h * d:(which % 3) * D + (h + 1) * d]
                    refp = src if which < 3 else oracle.rope3d(src, S, grid_w, 10000.0)
                    worst["qkv"] = max(worst["qkv"], oracle.rel_frobenius(g[h], refp))
    print("  " + ", ".join(f"{k} {v:.3e}" for k, v in worst.items()), flush=True)
    assert worst["y"] <= 5e-3 and worst["y_rounded"] <= 3e-3 and worst["qkv"] <= 5e-3, worst


@pytest.mark.parametrize("kw,grid_w,rule", [
    (dict(head_dim=64, heads=2, frames=12, tokens_per_frame=100, text_tokens=16), 10,
     "vdn_solve"),
    (dict(head_dim=128, heads=2, frames=7, tokens_per_frame=60, text_tokens=0, batch=2, chunk=3),
     6, "vdn_scaled"),   # a row tile spans both batch elements
    (dict(head_dim=64, heads=3, frames=9, tokens_per_frame=33, text_tokens=8), 11,
     "sana_scaled"),
])
def test_block_small(kw, grid_w, rule):
    _check(inputs.tiny_config(dtype="bf16", seed=140, rule=rule, **kw), grid_w, rule,
           check_qkv=True)


def test_block_full_width_guarded():
    # the full-size workloads' width: 24 heads of 128 (D = 3072), 832x480
    # frames (52 x 30 latent grid, 1,560 tokens), 6 frames; y poisoned and
    # guarded, the workspace guarded
    cfg = dict(inputs.WORKLOADS["clip-832x480-31f"], frames=6, name="clip-832x480-6f")
    _check(cfg, 52, guard=True, check_qkv=True)


def test_block_rejects_fp32_and_bad_grid():
    p = hwa.make_params(1, 2, 64, torch.float32)
    assert hwa.lib().hwa_block_workspace_bytes(4, 16, 2, ctypes.byref(p)) == 0
