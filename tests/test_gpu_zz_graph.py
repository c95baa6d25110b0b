"""Determinism and HIP-graph capture of hybrid_attn_fwd (needs an MI355X).

The library enqueues only kernels on the caller's stream (the softmax
kernel's work-queue counters are zeroed by the window-table kernel, not by a
memset), so a call can be captured in a graph and replayed. Every tile is
computed by the same instructions in the same order whichever workgroup takes
it from the work queues, so repeated calls and replays must agree bit for bit.
"""

import sys

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


@pytest.mark.parametrize("name", ["small-bf16-text", "tiny-f32"])
def test_softmax_bwd_repeat_and_graph_replay_bit_exact(name):
    # the backward enqueues only kernels too and has no atomics: each output
    # element is one fixed sum, so repeats and replays agree bit for bit
    from hybrid_window_softmax_amd import hwa
    from harness import to_dev
    cfg = inputs.WORKLOADS[name]
    _say(f"case {name}: softmax backward, eager calls, then a graph replayed three times")
    inp = inputs.make(cfg)
    bf = cfg["dtype"] == "bf16"
    q, k, v = (to_dev(getattr(inp, n), bf) for n in ("q", "k", "v"))
    g = to_dev(inputs.grad_output(cfg), bf)
    B, H, N, d = q.shape
    F, S, ch, r = cfg["frames"], cfg["tokens_per_frame"], cfg["chunk"], cfg["radius"]
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    o, _ = hwa.hybrid_attn_fwd(q, k, v, None, None, None, None, None, None, F, S, ch, r,
                               flags=hwa.FLAG_SOFTMAX_ONLY, softmax_lse=lse)
    ref = hwa.softmax_bwd(q, k, v, o, lse, g, F, S, ch, r)
    ws = ref[3]
    again = hwa.softmax_bwd(q, k, v, o, lse, g, F, S, ch, r, workspace=ws)
    torch.cuda.synchronize()

    def bits(t):
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t

    for x, y in zip(ref[:3], again[:3]):
        assert torch.equal(bits(x), bits(y))
    outs = [torch.empty_like(q) for _ in range(3)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        hwa.softmax_bwd(q, k, v, o, lse, g, F, S, ch, r, *outs, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hwa.softmax_bwd(q, k, v, o, lse, g, F, S, ch, r, *outs, workspace=ws)
    for rep in range(3):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        mism = sum(int((bits(a) != bits(b)).sum()) for a, b in zip(outs, ref[:3]))
        _say(f"  replay {rep}: {mism} elements differ from the eager call")
        assert mism == 0
    del graph


@pytest.mark.parametrize("name", ["small-bf16-text", "tiny-f32"])
def test_linear_bwd_graph_replay_bit_exact(name):
    # hwa_linear_bwd enqueues only kernels (no memsets, no atomics): a captured
    # call replays to the eager result bit for bit
    from hybrid_window_softmax_amd import hwa
    from harness import to_dev
    cfg = inputs.WORKLOADS[name]
    _say(f"case {name}: linear backward, eager call, then a graph replayed three times")
    inp = inputs.make(cfg)
    bf = cfg["dtype"] == "bf16"
    t = {n: to_dev(getattr(inp, n), bf) for n in
         ("q", "k", "v", "gate", "beta", "alpha", "conv_k", "conv_v", "rms_weight")}
    g = to_dev(inputs.grad_output(cfg), bf)
    st = to_dev(inputs.state_matrix(cfg), False)
    F, S, ch, r = cfg["frames"], cfg["tokens_per_frame"], cfg["chunk"], cfg["radius"]

    def call(grads=None, ws=None):
        return hwa.linear_bwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"], st,
                              t["conv_k"], t["conv_v"], g, F, S, ch, r, "vdn_solve", cfg["c"],
                              0.5, 1e-6, t["rms_weight"], grads=grads, workspace=ws)

    ref, ws = call()
    ref = {n: x.clone() for n, x in ref.items()}
    outs = {n: torch.empty_like(x) for n, x in ref.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(outs, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(outs, ws)

    def bits(x):
        return x.view(torch.int16) if x.dtype == torch.bfloat16 else x

    for rep in range(3):
        for x in outs.values():
            x.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        mism = sum(int((bits(outs[n]) != bits(ref[n])).sum()) for n in ref)
        _say(f"  replay {rep}: {mism} elements differ from the eager call")
        assert mism == 0
    del graph


def _graph_check(label, call, ref):
    """Capture `call` (which writes into its preallocated output and returns
    it) in a graph, replay it three times with eager work in between, and
    compare every replay with `ref` bit for bit."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one warm call on the capture stream
        out = call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = call()
    for r in range(3):
        out.fill_(0)               # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        mism = int((out.view(torch.int16) != ref.view(torch.int16)).sum())
        _say(f"  {label} replay {r}: {mism} elements differ from the eager call")
        assert mism == 0
    del graph


def test_routed_forward_graph_replay_bit_exact():
    # the routing kernels write every block mean, count and list entry the
    # softmax kernel reads: no memset, no atomics
    from hybrid_window_softmax_amd import hwa
    cfg = inputs.WORKLOADS["small-bf16-text"]
    _say("case small-bf16-text: routed forward (tau 0.5), eager calls, then a graph replayed")
    case = GpuCase(inputs.make(cfg))
    t = case.t

    def call(out=None, ws=None):
        return hwa.hybrid_attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"],
                                   case.text_state, t["conv_k"], t["conv_v"], cfg["frames"],
                                   cfg["tokens_per_frame"], cfg["chunk"], cfg["radius"],
                                   "vdn_solve", cfg["c"], 0.5, 1e-6, t["rms_weight"], out=out,
                                   workspace=ws, route_tau=0.5)

    ref, ws = call()
    again, _ = call(ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), again.view(torch.int16))
    out = torch.empty_like(ref)
    _graph_check("routed", lambda: call(out, ws)[0], ref)


def test_block_graph_replay_bit_exact():
    # the block's GEMMs and the attention enqueue only kernels
    from hybrid_window_softmax_amd import hwa
    from harness import to_dev
    cfg = inputs.tiny_config(head_dim=64, tokens_per_frame=64, frames=10, heads=2,
                             text_tokens=0, dtype="bf16", seed=170)
    _say("case block: eager calls, then a graph replayed")
    inp = inputs.make(cfg)
    xb, wqb, wob = inputs.block_inputs(cfg)
    t = {n: to_dev(getattr(inp, n), True) for n in
         ("beta", "alpha", "gate", "conv_k", "conv_v", "rms_weight")}
    x, wq, wo = (to_dev(a, True) for a in (xb, wqb, wob))

    def call(y=None, ws=None):
        return hwa.block_fwd(x, wq, wo, t["beta"], t["alpha"], t["gate"], None, t["conv_k"],
                             t["conv_v"], cfg["heads"], cfg["frames"], cfg["tokens_per_frame"],
                             8, 10000.0, cfg["chunk"], cfg["radius"], "vdn_solve", cfg["c"],
                             0.5, 1e-6, t["rms_weight"], y=y, workspace=ws)

    ref, ws = call()
    again, _ = call(ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), again.view(torch.int16))
    y = torch.empty_like(ref)
    _graph_check("block", lambda: call(y, ws)[0], ref)
