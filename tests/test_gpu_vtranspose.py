"""The transposed v that the softmax kernel streams (workspace region v_t,
[B, H, d, round_up64(N)] bf16 with zeros past N), compared bit for bit with v
transposed after the whole workspace was filled with NaN bytes. On bf16
forward calls whose frames hold a multiple of 4 tokens the statistics kernel
writes it while it reads v for the linear branch; frames of other sizes and
softmax-only calls use the separate transpose kernel. Both must leave the same
bytes (include/hwa.h documents the workspace layout)."""
import sys

import pytest
import torch

from hybrid_window_softmax_amd import hwa, inputs
from harness import GpuCase, ws_view

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,d,flags", [
    (24, 128, 0),                       # statistics kernel, keys past N padded
    (100, 64, 0),                       # statistics kernel, d 64
    (64, 128, 0),                       # statistics kernel, N a multiple of 64
    (33, 128, 0),                       # separate transpose (S % 4 != 0)
    (24, 64, hwa.FLAG_SOFTMAX_ONLY),    # separate transpose (no linear branch)
])
def test_transposed_v_bit_exact(S, d, flags):
    cfg = inputs.tiny_config(frames=7, text_tokens=8, head_dim=d, tokens_per_frame=S,
                             dtype="bf16", heads=2, batch=2, seed=131)
    print(f"case S={S} d={d} flags={flags}", flush=True)
    sys.stdout.flush()
    case = GpuCase(inputs.make(cfg))
    L = case.layout()
    ws = torch.full((L["total"],), 0xFF, dtype=torch.uint8, device="cuda")
    case.run("vdn_solve", flags, True, workspace=ws)
    torch.cuda.synchronize()
    B, H, F = cfg["batch"], cfg["heads"], cfg["frames"]
    N = F * S
    Np = -(-N // 64) * 64
    got = ws_view(ws, L["v_t"], (B, H, d, Np), torch.bfloat16).cpu()
    want = torch.zeros(B, H, d, Np, dtype=torch.bfloat16)
    want[..., :N] = case.t["v"].cpu().transpose(-1, -2)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
