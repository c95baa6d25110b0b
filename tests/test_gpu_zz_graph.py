"""Determinism and HIP-graph capture of hybrid_attn_fwd (needs an MI355X).

The library enqueues only kernels on the caller's stream (the softmax
kernel's work-queue counters are zeroed by the window-table kernel, not by a
memset), so a call can be captured in a graph and replayed. Every tile is
computed by the same instructions in the same order whichever workgroup takes
it from the work queues, so repeated calls and replays must agree bit for bit.
"""

import sys

import numpy as np
import pytest
import torch

from hybrid_window_softmax_amd import inputs
from harness import GpuCase

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", ["small-bf16-text", "tiny-f32"])
def test_repeat_and_graph_replay_bit_exact(name):
    cfg = inputs.WORKLOADS[name]
    _say(f"case {name}: eager calls, then a captured graph replayed three times")
    case = GpuCase(inputs.make(cfg))
    rule = cfg["rules"][0]
    text = cfg["text_tokens"] > 0
    ref, ws = case.run(rule, 0, text)
    again, _ = case.run(rule, 0, text, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref,
                       again.view(torch.int16) if again.dtype == torch.bfloat16 else again)

    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one warm call on the capture stream
        case.run(rule, 0, text, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        case.run(rule, 0, text, out=out, workspace=ws)
    for r in range(3):
        out.fill_(0)               # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        a = out.view(torch.int16) if out.dtype == torch.bfloat16 else out
        b = ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref
        mism = int((a != b).sum())
        _say(f"  replay {r}: {mism} elements differ from the eager call")
        assert mism == 0
    del graph
