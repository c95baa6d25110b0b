"""hybrid_attn_fwd_noalloc (the forward on the library's fixed scratch array,
for callers that cannot allocate) against hybrid_attn_fwd (the same kernels on
a caller-owned workspace), through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input: each
output must equal the workspace entry point's bit for bit (the same kernels
on the same data; nothing a call reads from the scratch array is left over
from the previous call), and so lie within the parity bar of the oracle
comparisons of the forward. fp32 and bf16 (fused readout) calls, with the
softmax branch's lse and output requested on one of them.
"""

import pytest
import torch

from hybrid_window_softmax_amd import hwa, inputs
from harness import GpuCase

pytestmark = pytest.mark.gpu


def _run(cfg, noalloc, rule="vdn_solve", with_sm=False):
    inp = inputs.make(cfg)
    case = GpuCase(inp)
    t = case.t
    c = inp.cfg
    B, H, N, d = t["q"].shape
    kw = {}
    if with_sm:
        kw = dict(softmax_lse=torch.empty((B, H, N), dtype=torch.float32, device="cuda"),
                  softmax_out=torch.empty_like(t["q"]))
    out, ws = hwa.hybrid_attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"],
                                  case.text_state, t["conv_k"], t["conv_v"], c["frames"],
                                  c["tokens_per_frame"], c["chunk"], c["radius"], rule, c["c"],
                                  0.5, 1e-6, t["rms_weight"], noalloc=noalloc, **kw)
    torch.cuda.synchronize()
    if noalloc:
        assert ws is None
    res = [out]
    if with_sm:
        res += [kw["softmax_lse"], kw["softmax_out"]]
    return res


@pytest.mark.parametrize("first,second,rule", [
    ("small-bf16-text",
     inputs.tiny_config(frames=7, text_tokens=8, head_dim=64, tokens_per_frame=33,
                        dtype="bf16", heads=3, seed=106, chunk=3), "vdn_solve"),
    (inputs.tiny_config(frames=17, text_tokens=16, head_dim=64, tokens_per_frame=24, heads=2,
                        seed=121),
     inputs.tiny_config(frames=11, text_tokens=8, head_dim=32, tokens_per_frame=10,
                        seed=122), "vdn_scaled"),
])
def test_noalloc_matches_workspace_entry_point(first, second, rule):
    for i, cfg in enumerate((first, second)):
        cfg = inputs.WORKLOADS[cfg] if isinstance(cfg, str) else cfg
        print(f"case noalloc call {i + 1}: {cfg['name']} {cfg['dtype']} H{cfg['heads']} "
              f"d{cfg['head_dim']} F{cfg['frames']} S{cfg['tokens_per_frame']} {rule}",
              flush=True)
        with_sm = i == 0
        ref = _run(cfg, False, rule, with_sm)
        got = _run(cfg, True, rule, with_sm)
        for r, g in zip(ref, got):
            assert bool(torch.isfinite(g.float()).all())
            assert torch.equal(r, g), float((r.float() - g.float()).abs().max())
