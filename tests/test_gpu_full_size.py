"""Full-size parity of hybrid_attn_fwd in the launch configuration the
benchmark times (bf16, both branches, the linear-branch readout fused into
the softmax kernel's epilogue), at 48,360, 132,600 and 262,144 tokens.

Per workload and rule:
- whole heads: the fused `out` of whole heads is compared with the oracle's
  o_sm + y over all N tokens (max relative Frobenius error over the heads
  checked, as for the small cases), and `softmax_out`, the log-sum-exp and the
  HWA_FLAG_LINEAR_ONLY y of the same heads with their oracle values;
- every head: `out` - `softmax_out` against the LINEAR_ONLY y on the GPU
  (relative Frobenius per head), o_sm on sampled query rows (chunk edges,
  tile edges, random rows) against the oracle, and the log-sum-exp on the
  same rows;
- every output is pre-filled with NaN inside guard bands of NaN, and the
  workspace sits between bands of 0xA5 bytes: after the call every element is
  finite (nothing left unwritten) and every guard is untouched (nothing
  written past a buffer).
The call without softmax_out / lse (the benchmark's) and the call with them
must give the same `out` bit for bit.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from hybrid_window_softmax_amd import hwa, inputs
from harness import (TOL, GpuCase, check_poisoned, check_workspace_guard, guarded_workspace,
                     oracle_linear_head, oracle_text_state, out_f64, poisoned, sample_rows)

pytestmark = pytest.mark.gpu

LSE_TOL = 4e-3  # absolute, natural-log units (bf16 q, k)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _full_size(name, rules, heads_full):
    cfg = inputs.WORKLOADS[name]
    _say(f"case {name}: generating inputs")
    inp = inputs.make(cfg)
    case = GpuCase(inp)
    B, H, d = cfg["batch"], cfg["heads"], cfg["head_dim"]
    F, S, ch, r = cfg["frames"], cfg["tokens_per_frame"], cfg["chunk"], cfg["radius"]
    N = F * S
    tol = TOL[cfg["dtype"]]
    rows = sample_rows(cfg)
    lo, hi = oracle.window_bounds(F, ch, r)
    p = hwa.make_params(B, H, d, torch.bfloat16)
    need = hwa.workspace_bytes(F, S, ch, p)
    # the softmax branch does not depend on the rule: oracle values once per head
    o_sm_ref = {}
    lse_ref = {}
    for h in heads_full:
        _say(f"  oracle softmax branch, head {h}")
        q64, k64, v64 = inp.f64("q", 0, h), inp.f64("k", 0, h), inp.f64("v", 0, h)
        o_sm_ref[h] = oracle.softmax_branch(q64, k64, v64, S, lo, hi)
        lse_ref[h] = oracle.softmax_lse(q64, k64, S, lo, hi)
    for rule in rules:
        _say(f"case {name} rule={rule}")
        ws, ws_flat = guarded_workspace(need)
        out, out_flat = poisoned((B, H, N, d), torch.bfloat16)
        sm, sm_flat = poisoned((B, H, N, d), torch.bfloat16)
        lse, lse_flat = poisoned((B, H, N), torch.float32)
        y, y_flat = poisoned((B, H, N, d), torch.bfloat16)
        bench_out, bo_flat = poisoned((B, H, N, d), torch.bfloat16)
        t = case.t
        common = (t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"], case.text_state,
                  t["conv_k"], t["conv_v"], F, S, ch, r, rule, cfg["c"], 0.5, 1e-6,
                  t["rms_weight"])
        hwa.hybrid_attn_fwd(*common, out=bench_out, workspace=ws)          # as timed
        hwa.hybrid_attn_fwd(*common, out=out, workspace=ws, softmax_lse=lse, softmax_out=sm)
        hwa.hybrid_attn_fwd(*common, out=y, workspace=ws, flags=hwa.FLAG_LINEAR_ONLY)
        torch.cuda.synchronize()
        for v, fl, nm in ((bench_out, bo_flat, "out (bench call)"), (out, out_flat, "out"),
                          (sm, sm_flat, "softmax_out"), (lse, lse_flat, "lse"),
                          (y, y_flat, "y (LINEAR_ONLY)")):
            check_poisoned(v, fl, f"{name} {rule} {nm}")
        check_workspace_guard(ws_flat, need, f"{name} {rule}")
        assert torch.equal(bench_out.view(torch.int16), out.view(torch.int16)), \
            "out differs between the calls with and without softmax_out / lse"
        # every head, on the GPU: out - o_sm is the linear branch
        lin = (out.float() - sm.float()).view(B * H, -1)
        yf = y.float().view(B * H, -1)
        e_split = ((lin - yf).norm(dim=1) / yf.norm(dim=1)).max().item()
        # every head: sampled rows of o_sm and of the log-sum-exp
        idx = torch.from_numpy(rows).to(out.device)
        s_rows = sm[0].index_select(1, idx).float().cpu().numpy().astype(np.float64)
        l_rows = lse[0].index_select(1, idx).cpu().numpy().astype(np.float64)
        e_rows = 0.0
        e_lse_rows = 0.0
        for h in range(H):
            q32, k32 = inp.f32("q", 0, h), inp.f32("k", 0, h)
            ref = oracle.softmax_rows(q32, k32, inp.f32("v", 0, h), S, lo, hi, rows)
            e_rows = max(e_rows, oracle.rel_frobenius(s_rows[h], ref))
            ref_l = oracle.softmax_lse_rows(q32, k32, S, lo, hi, rows)
            e_lse_rows = max(e_lse_rows, np.abs(l_rows[h] - ref_l).max())
        # whole heads
        worst = {"out": 0.0, "o_sm": 0.0, "y": 0.0, "lse": 0.0}
        for h in heads_full:
            _say(f"  oracle linear branch, head {h}")
            y_ref, _ = oracle_linear_head(inp, 0, h, rule)
            worst["out"] = max(worst["out"], oracle.rel_frobenius(out_f64(out[0, h]),
                                                                  o_sm_ref[h] + y_ref))
            worst["o_sm"] = max(worst["o_sm"], oracle.rel_frobenius(out_f64(sm[0, h]), o_sm_ref[h]))
            worst["y"] = max(worst["y"], oracle.rel_frobenius(out_f64(y[0, h]), y_ref))
            worst["lse"] = max(worst["lse"], np.abs(lse[0, h].cpu().numpy() - lse_ref[h]).max())
        _say(f"  {rule}: whole heads {list(heads_full)}: " +
             ", ".join(f"{k} {v:.3e}" for k, v in worst.items()) +
             f"; all heads: out - o_sm vs y {e_split:.3e}, o_sm rows {e_rows:.3e}, "
             f"lse rows {e_lse_rows:.3e}")
        for k in ("out", "o_sm", "y"):
            assert worst[k] <= tol, f"{name} {rule} {k}: {worst[k]:.3e} > {tol:g}"
        assert worst["lse"] <= LSE_TOL and e_lse_rows <= LSE_TOL, (worst["lse"], e_lse_rows)
        assert e_split <= tol, f"{name} {rule} out - o_sm vs y: {e_split:.3e}"
        assert e_rows <= tol, f"{name} {rule} o_sm rows: {e_rows:.3e}"
        del out, sm, lse, y, bench_out, ws, out_flat, sm_flat, lse_flat, y_flat, bo_flat, ws_flat
        torch.cuda.empty_cache()


def test_clip_48360tok_whole_heads():
    _full_size("clip-832x480-31f", ("vdn_solve",), (0, 23))


def test_long_clip_132600tok_whole_heads_all_rules():
    _full_size("long-clip-832x480-85f", oracle.RULES, (0, 23))


def test_canvas_262144tok_whole_head():
    _full_size("canvas-1024x1024-64f", ("vdn_solve",), (23,))


def test_text_state_full_size_guarded():
    # hwa_text_state at the full workloads' shape (24 heads, d 128, 256 text
    # tokens): the state poisoned and guarded, the workspace guarded, every
    # head against the oracle
    cfg = inputs.WORKLOADS["long-clip-832x480-85f"]
    inp = inputs.make(dict(cfg, frames=1, tokens_per_frame=1))  # text tokens only matter
    B, H, d, T = cfg["batch"], cfg["heads"], cfg["head_dim"], cfg["text_tokens"]
    _say(f"case text state B{B} H{H} d{d} T{T}, guarded")
    kt, vt, bt = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
                  if a.dtype == np.uint16 else torch.from_numpy(a).cuda()
                  for a in (inp.k_txt, inp.v_txt, inp.beta_txt))
    st, st_flat = poisoned((B, H, d, d), torch.float32)
    p = hwa.make_params(B, H, d, torch.bfloat16)
    need = int(hwa.lib().hwa_text_state_workspace_bytes(T, ctypes.byref(p)))
    ws, ws_flat = guarded_workspace(need)
    hwa.text_state(kt, vt, bt, workspace=ws, out=st)
    torch.cuda.synchronize()
    check_poisoned(st, st_flat, "text state")
    check_workspace_guard(ws_flat, need, "text state")
    got = st.cpu().numpy()
    worst = max(oracle.rel_frobenius(got[0, h], oracle_text_state(inp, 0, h)) for h in range(H))
    _say(f"  max rel Frobenius {worst:.3e}")
    assert worst < 1e-5, worst
