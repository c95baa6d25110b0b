"""GPU parity of the block-sparse routed softmax branch (HWA_FLAG_ROUTED) with
the routing oracle (oracle.routed_softmax), through the C ABI.

The routing decisions are floating-point comparisons (fp32 on the GPU, fp64
in the oracle), so a block whose score lies within rounding of the threshold
may go either way: every decision farther from the threshold than a small
margin must match the oracle's, the first best block must be kept, and the
output is then compared with the oracle's routed softmax on the GPU's own
kept blocks (5e-3, the bf16 bar). With tau = -inf every block is kept and the
routed kernel must reproduce the dense one bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from hybrid_window_softmax_amd import hwa, inputs
from harness import (GpuCase, check_poisoned, check_workspace_guard, guarded_workspace,
                     out_f64, poisoned)

pytestmark = pytest.mark.gpu


def _run(case, route_tau, flags=hwa.FLAG_SOFTMAX_ONLY, guard=False):
    c = case.cfg
    t = case.t
    out = ws = None
    if guard:
        B, H, N, d = t["q"].shape
        out, out_flat = poisoned((B, H, N, d), torch.bfloat16)
        p = hwa.make_params(B, H, d, torch.bfloat16, flags=flags | hwa.FLAG_ROUTED)
        need = hwa.workspace_bytes(c["frames"], c["tokens_per_frame"], c["chunk"], p)
        ws, ws_flat = guarded_workspace(need)
    o, ws = hwa.hybrid_attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"],
                                case.text_state, t["conv_k"], t["conv_v"], c["frames"],
                                c["tokens_per_frame"], c["chunk"], c["radius"], "vdn_solve",
                                c["c"], 0.5, 1e-6, t["rms_weight"], flags=flags, out=out,
                                workspace=ws, route_tau=route_tau)
    torch.cuda.synchronize()
    if guard:
        check_poisoned(o, out_flat, "routed out")
        check_workspace_guard(ws_flat, need, "routed")
    return o, ws


def _lists(case, ws):
    c = case.cfg
    B, H = c["batch"], c["heads"]
    p = hwa.make_params(B, H, c["head_dim"], torch.bfloat16, flags=hwa.FLAG_ROUTED)
    L = hwa.route_layout(c["frames"], c["tokens_per_frame"], c["chunk"], p)
    nch = -(-c["frames"] // c["chunk"])
    tpc, stride = L["tiles_per_chunk"], L["stride"]
    cnt = ws[L["count"]:L["count"] + B * H * nch * tpc * 4].view(torch.int32)
    lst = ws[L["list"]:L["list"] + B * H * nch * tpc * stride * 2].view(torch.int16)
    cnt = cnt.cpu().numpy().reshape(B, H, nch, tpc)
    lst = lst.cpu().numpy().view(np.uint16).reshape(B, H, nch, tpc, stride)
    return cnt, lst


def _check(cfg, tau, heads_full=None, guard=False):
    print(f"case routed {cfg['name']} H{cfg['heads']} d{cfg['head_dim']} F{cfg['frames']} "
          f"S{cfg['tokens_per_frame']} chunk {cfg['chunk']} tau {tau}", flush=True)
    inp = inputs.make(cfg)
    case = GpuCase(inp)
    o, ws = _run(case, tau, guard=guard)
    cnt, lst = _lists(case, ws)
    got = out_f64(o)
    B, H, S = cfg["batch"], cfg["heads"], cfg["tokens_per_frame"]
    nch = -(-cfg["frames"] // cfg["chunk"])
    tpc = cnt.shape[3]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads_full is None else heads_full
    worst, kept, total, near = 0.0, 0, 0, 0
    for b, h in heads:
        q, k, v = inp.f64("q", b, h), inp.f64("k", b, h), inp.f64("v", b, h)
        tiles = oracle.route_scores(q, k, S, cfg["chunk"], cfg["radius"])
        masks = []
        ti = 0
        for ci in range(nch):
            qb = ci * cfg["chunk"] * S
            for t in range(tpc):
                if ti >= len(tiles) or tiles[ti][0] != qb + 256 * t:
                    continue
                _, _, blocks, s = tiles[ti]
                ti += 1
                n = int(cnt[b, h, ci, t])
                gl = lst[b, h, ci, t, :n].astype(np.int64)
                assert n >= 1 and np.all(np.diff(gl) > 0) and gl[-1] < len(blocks), (ci, t, gl)
                m = np.zeros(len(blocks), dtype=bool)
                m[gl] = True
                thr = s.mean() + tau * s.std() if np.isfinite(tau) else -np.inf
                ref = oracle.route_keep(s, tau)
                margin = 1e-5 * (abs(thr) + s.std() + np.abs(s).max()) if np.isfinite(tau) else 0
                far = np.abs(s - thr) > margin
                assert np.array_equal(m[far], ref[far]), (b, h, ci, t)
                best = s.max()
                assert m[np.abs(s - best) <= margin].any(), "the best block must be kept"
                near += int((~far).sum())
                kept += n
                total += len(blocks)
                masks.append(m)
        assert ti == len(tiles)
        o_ref, _ = oracle.routed_softmax(q, k, v, S, cfg["chunk"], cfg["radius"], tau, keep=masks)
        worst = max(worst, oracle.rel_frobenius(got[b, h], o_ref))
    print(f"  o_sm max rel Frobenius {worst:.3e}; kept {kept} of {total} blocks "
          f"({kept / total:.3f}), {near} within rounding of the threshold", flush=True)
    assert worst <= 5e-3, worst
    return kept / total


@pytest.mark.parametrize("kw", [
    dict(head_dim=128, tokens_per_frame=100, frames=12, heads=2, text_tokens=16),
    dict(head_dim=64, tokens_per_frame=256, frames=20, heads=2, text_tokens=0, chunk=3),
    dict(head_dim=128, tokens_per_frame=33, frames=9, heads=1, text_tokens=0, radius=2),
])
def test_routed_keep_all_is_the_dense_kernel(kw):
    # tau = -inf keeps every block: the routed kernel visits the dense tiles
    cfg = inputs.tiny_config(dtype="bf16", seed=150, **kw)
    print(f"case routed keep-all {cfg['name']} d{cfg['head_dim']} S{cfg['tokens_per_frame']}",
          flush=True)
    case = GpuCase(inputs.make(cfg))
    for flags in (hwa.FLAG_SOFTMAX_ONLY, 0):
        dense, _ = case.run("vdn_solve", flags)
        routed, _ = _run(case, -math.inf, flags)
        assert torch.equal(dense.view(torch.int16), routed.view(torch.int16)), flags


@pytest.mark.parametrize("tau", [0.0, 1.2, 2.0])
def test_routed_small(tau):
    cfg = inputs.tiny_config(head_dim=128, tokens_per_frame=200, frames=17, heads=2,
                             text_tokens=0, dtype="bf16", seed=151)
    _check(cfg, tau)


def test_routed_full_size_guarded():
    # the 132,600-token workload at the report's middle threshold: every head
    # on the GPU (output poisoned and guarded), two whole heads against the
    # oracle
    _check(inputs.WORKLOADS["long-clip-832x480-85f"], 1.5, heads_full=[(0, 0), (0, 23)],
           guard=True)


@pytest.mark.parametrize("kw,tau", [
    (dict(head_dim=128, tokens_per_frame=100, frames=1), 1.0),                 # one frame
    (dict(head_dim=64, tokens_per_frame=1, frames=23, chunk=4), 0.5),          # one token a frame
    (dict(head_dim=128, tokens_per_frame=300, frames=8, radius=0), 1.5),       # no neighbours
    (dict(head_dim=64, tokens_per_frame=130, frames=11, chunk=1), 10.0),       # best block only
    (dict(head_dim=128, tokens_per_frame=77, frames=9, batch=2, heads=2), -0.5),
])
def test_routed_edge_shapes(kw, tau):
    cfg = inputs.tiny_config(text_tokens=0, dtype="bf16", seed=152, **kw)
    _check(cfg, tau)
