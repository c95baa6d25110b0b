#!/usr/bin/env python3
"""Benchmark of the hybrid window-softmax attention forward on one MI355X.

One step = one hybrid_attn_fwd call over the whole workload (window table,
V transpose, windowed softmax, fused features + statistics, update maps,
bidirectional scan, readout epilogue), inputs resident in HBM. Prints one
JSON line: whole-job tokens/s, per-kernel times from hipEvents the library
records at its kernel boundaries on the call's stream, the roofline of the
dominant kernel (the windowed softmax, bf16 MFMA) and the fp64 CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload long-clip-832x480-85f] [--rule vdn_solve]

With --softmax-bwd it instead times the backward of the windowed softmax
branch (hwa_softmax_bwd: dq, dk, dv from q, k, v, the branch output, its
log-sum-exp and the upstream gradient) on the same workload and prints that
line; with --linear-bwd, the backward of the linear branch (hwa_linear_bwd:
every input's gradient, fp32 arithmetic); with --train-step, the forward
followed by both backward passes (every input's gradient of the output).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (vector, packed) / fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "softmax_traffic.json")
# the workload the softmax kernel's HBM counters were taken on
TRAFFIC_WORKLOAD = "long-clip-832x480-85f"
# the full-size workloads the metric spans (48k to 262k tokens)
RANGE_WORKLOADS = ("clip-832x480-31f", "long-clip-832x480-85f", "canvas-1024x1024-64f")
# latent grid width of the workloads' frames (832x480: 52 x 30; 1024x1024: 64 x 64)
BLOCK_GRID_W = {1560: 52, 4096: 64, 256: 16, 16: 4}
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "softmax_bwd_traffic.json")
# the softmax kernel's sources (the kernel, the readout epilogue and the tile
# helpers it includes)
SOFTMAX_SRCS = [os.path.join(ROOT, "hybrid_window_softmax_amd", "csrc", n)
                for n in ("softmax.hip", "readout_core.h", "attn_tile.h", "hwa_internal.h")]
# the backward kernels' sources
SOFTMAX_BWD_SRCS = [os.path.join(ROOT, "hybrid_window_softmax_amd", "csrc", n)
                    for n in ("softmax_bwd.hip", "attn_tile.h", "hwa_internal.h")]
LIN_BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "linear_bwd_traffic.json")
LIN_BWD_SRCS = [os.path.join(ROOT, "hybrid_window_softmax_amd", "csrc", n)
                for n in ("linear_bwd.hip", "linear_bwd.h", "hwa_internal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def window_pairs(cfg):
    """Query-key token pairs one head scores: sum_t S * S * (hi_t - lo_t + 1)."""
    F, S, ch, r = cfg["frames"], cfg["tokens_per_frame"], cfg["chunk"], cfg["radius"]
    tot = 0
    for t in range(F):
        c = t // ch
        lo, hi = max(0, (c - r) * ch), min(F - 1, (c + r + 1) * ch - 1)
        tot += S * S * (hi - lo + 1)
    return tot


def algorithmic_work(cfg):
    """Algorithmic bytes and flops of every kernel of one call (bf16 I/O)."""
    B, H, d = cfg["batch"], cfg["heads"], cfg["head_dim"]
    F, S = cfg["frames"], cfg["tokens_per_frame"]
    N = F * S
    nch = -(-F // cfg["chunk"])
    io = 2 if cfg["dtype"] == "bf16" else 4
    tok = B * H * N            # (token, head) units
    mat = B * H * F * d * d * 4  # one fp32 [B,H,F,d,d] tensor
    bank = B * H * (nch + 1) * d * d * 4
    return {
        "vtranspose": dict(bytes=2 * tok * d * io, flops=0),
        "softmax": dict(bytes=4 * tok * d * io, flops=4 * d * window_pairs(cfg) * B * H),
        "stats": dict(bytes=2 * tok * d * io + tok * 4 + 2 * mat, flops=4 * d * d * tok),
        "inverse": dict(bytes=2 * mat, flops=2 * d * d * d * B * H * F),
        "scan": dict(bytes=4 * mat + 2 * B * H * F * d * 4 + 2 * bank,
                     flops=2 * 2 * d * d * d * B * H * F),
        # decay products, then S_t of every frame (reads both gathered bank
        # states and the decays, writes fp16 S_t)
        "decay+state": dict(bytes=B * H * F * (3 * d * 4 + 2 * d * d * 4 + 2 * d * 4 + d * d * 2),
                            flops=3 * d * d * B * H * F),
        "readout": dict(bytes=4 * tok * d * io + B * H * F * d * d * 2, flops=2 * d * d * tok),
        # bf16 calls fuse the readout into the softmax kernel's epilogue: q and
        # out are not re-read, the gate and S_t are
        "softmax+readout": dict(bytes=4 * tok * d * io + tok * d * io + B * H * F * d * d * 2,
                                flops=4 * d * window_pairs(cfg) * B * H + 2 * d * d * tok),
    }


def sources_sha256(paths=None):
    """sha256 over a kernel's source files, in order (default: the forward
    softmax kernel's)."""
    h = hashlib.sha256()
    for path in paths or SOFTMAX_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def softmax_sources_sha256():
    return sources_sha256(SOFTMAX_SRCS)


def recorded_traffic(path=TRAFFIC_FILE, srcs=None):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary, or None when the kernel's sources changed since it was taken."""
    try:
        with open(path) as f:
            rec = json.load(f)
        sha = sources_sha256(srcs or SOFTMAX_SRCS)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def softmax_traffic():
    return recorded_traffic(TRAFFIC_FILE, SOFTMAX_SRCS)


def linear_bwd_traffic(kernel):
    """HBM bytes per launch of one linear-backward kernel from the committed
    counter summary (which covers several kernels), or None when the sources
    changed since the counters were taken."""
    try:
        with open(LIN_BWD_TRAFFIC_FILE) as f:
            rec = json.load(f)
        sha = sources_sha256(LIN_BWD_SRCS)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("kernels", {}).get(kernel, {}).get("bytes_per_launch")


def host_info():
    """CPU model and the numpy / BLAS build this process uses."""
    import numpy as np
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')})"
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "numpy": np.__version__, "blas": blas}


def cpu_workers():
    """Worker processes for the oracle: the host cores this process may run
    on, at most 16 (one GPU's share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(inp, rule, heads_run=None, workers=None):
    """The fp64 oracle as it stands (oracle.hybrid_attn: softmax branch per
    (batch, head, query chunk), linear branch per (batch, head), text states)
    on the first `heads_run` heads of the same workload, run by a pool of
    `workers` processes with one BLAS thread each, scaled to the whole job's
    tokens/s. Call it before the GPU is touched: the pool forks."""
    import math

    import numpy as np
    import oracle
    cfg = inp.cfg
    W = workers or cpu_workers()
    F, S, ch = cfg["frames"], cfg["tokens_per_frame"], cfg["chunk"]
    nch = -(-F // ch)
    if heads_run is None:  # enough tasks for six per worker (about 10-20 s)
        heads_run = max(1, math.ceil(6 * W / (nch + 1)))
    hr = min(heads_run, cfg["heads"])
    B = cfg["batch"]
    from hybrid_window_softmax_amd import inputs

    def f32(name):  # exact upcast of the first hr heads of an I/O tensor
        a = np.ascontiguousarray(getattr(inp, name)[:, :hr])
        return inputs.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a

    q, k, v, gate = f32("q"), f32("k"), f32("v"), f32("gate")
    t0 = time.perf_counter()
    st = None
    if inp.k_txt is not None:
        st = np.stack([np.stack([oracle.text_state(inp.f64("k_txt", b, h),
                                                   inp.f64("v_txt", b, h),
                                                   inp.beta_txt[b, h].astype(np.float64))
                                 for h in range(hr)]) for b in range(B)])
    oracle.hybrid_attn(q, k, v, inp.beta[:, :hr], inp.alpha[:, :hr], gate, st,
                       inp.conv_k[:hr], inp.conv_v[:hr], inp.rms_weight, F, S, ch,
                       cfg["radius"], rule, cfg["c"], 0.5, 1e-6, workers=W)
    dt = time.perf_counter() - t0
    N = F * S
    total_s = dt * cfg["heads"] / hr
    return {"value": N * B / total_s, "unit": "tokens/s", "cores": W, "kind": "oracle",
            "sample": f"{hr} of {cfg['heads']} heads (all {N} tokens of each; "
                      f"{B * hr * (nch + 1)} tasks: softmax per (batch, head, query chunk), "
                      f"linear branch per (batch, head), plus the text states) on {W} worker "
                      f"processes with one BLAS thread each, {dt:.1f} s wall, scaled by heads",
            **host_info()}


def softmax_bwd_cpu_baseline(inp, g_host, heads_run=1):
    """The oracle's windowed-softmax gradient on `heads_run` whole heads,
    scaled to the whole job's tokens/s."""
    import numpy as np
    import oracle
    from hybrid_window_softmax_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    cfg = inp.cfg
    S = cfg["tokens_per_frame"]
    lo, hi = oracle.window_bounds(cfg["frames"], cfg["chunk"], cfg["radius"])
    t0 = time.perf_counter()
    for h in range(heads_run):
        g = inputs.bf16_bits_to_f32(g_host[0, h]) if g_host.dtype == np.uint16 else g_host[0, h]
        oracle.softmax_branch_grad(inp.f64("q", 0, h), inp.f64("k", 0, h), inp.f64("v", 0, h),
                                   g.astype(np.float64), S, lo, hi)
    dt = time.perf_counter() - t0
    N = cfg["frames"] * S
    total_s = dt * cfg["heads"] * cfg["batch"] / heads_run
    return {"value": N * cfg["batch"] / total_s, "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{heads_run} of {cfg['heads']} heads (all {N} tokens of each), "
                      f"{dt:.1f} s wall, scaled by heads"}


def bench_softmax_bwd(args, cfg, inp, up):
    """One step = one hwa_softmax_bwd over the whole workload (inputs, the
    branch output and its log-sum-exp resident in HBM)."""
    import torch
    from hybrid_window_softmax_amd import hwa, inputs
    g_host = inputs.grad_output(cfg)
    q, k, v, g = up(inp.q), up(inp.k), up(inp.v), up(g_host)
    F, S = cfg["frames"], cfg["tokens_per_frame"]
    B, H, N, d = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    o, ws_f = hwa.hybrid_attn_fwd(q, k, v, None, None, None, None, None, None, F, S,
                                  cfg["chunk"], cfg["radius"], flags=hwa.FLAG_SOFTMAX_ONLY,
                                  softmax_lse=lse)
    del ws_f
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def call(events=None, ws=None):
        return hwa.softmax_bwd(q, k, v, o, lse, g, F, S, cfg["chunk"], cfg["radius"], dq=dq,
                               dk=dk, dv=dv, workspace=ws, stage_events=events)[3]

    log("bench: softmax backward warmup")
    ws = call()
    for _ in range(max(0, args.warmup - 1)):
        call(ws=ws)
    torch.cuda.synchronize()
    timer = hwa.StageTimer(args.steps, hwa.NUM_BWD_STAGE_EVENTS, hwa.BWD_STAGES)
    log(f"bench: timing {args.steps} backward steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(events=timer.sets[i], ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage = timer.stage_ms()
    timer.close()
    ms = (t1 - t0) * 1000.0 / args.steps
    log("bench: stage ms " + ", ".join(f"{k} {v:.3f}" for k, v in stage.items()))
    pairs = window_pairs(cfg) * B * H
    io = 2 if cfg["dtype"] == "bf16" else 4
    tok = B * H * N
    # executed products per query-key pair: dq recomputes S and dP and forms
    # dQ (3 x 2d flop); dk/dv recomputes S and dP and forms dV and dK (4 x 2d)
    work = {
        # read o, g and lse, write delta and lse2
        "prep": dict(bytes=tok * (2 * d * io + 4 + 8), flops=0),
        "dq": dict(bytes=0, flops=6 * d * pairs),
        "dkdv": dict(bytes=0, flops=8 * d * pairs),
    }
    kernels = {}
    for name, w in work.items():
        sec = stage[name] / 1000.0
        rec = {"ms": round(stage[name], 4)}
        if w["bytes"]:
            rec["hbm_GBs"] = round(w["bytes"] / sec / 1e9, 1)
            rec["hbm_frac"] = round(w["bytes"] / sec / 1e9 / PEAK_HBM_GBS, 4)
        if w["flops"]:
            rec["TFLOPs"] = round(w["flops"] / sec / 1e12, 2)
            rec["frac"] = round(w["flops"] / sec / 1e12 / PEAK_BF16_TFLOPS, 4)
        kernels[name] = rec
    dom = "dkdv"
    achieved = work[dom]["flops"] / (stage[dom] / 1000.0) / 1e12
    roofline = {"kernel": "softmax_bwd_dkdv_kernel", "bound": "mfma",
                "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(BWD_TRAFFIC_FILE, SOFTMAX_BWD_SRCS),
                "algorithmic_flops_per_launch": work[dom]["flops"]}
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle's gradient on a sample")
        del q, k, v, g, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
        cpu = softmax_bwd_cpu_baseline(inp, g_host, args.cpu_heads or 1)
    return {
        "metric": "windowed-softmax backward (dq, dk, dv) tokens/s",
        "value": round(B * N / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: B{B} H{H} d{d} F{F} x S{S} = {N} tokens, "
                               f"chunk {cfg['chunk']} radius {cfg['radius']}, softmax branch "
                               f"backward",
                   "tokens": N, "heads": H, "head_dim": d},
        # the method's five products per pair (S, dP, dV, dK, dQ), over the step
        "algorithmic_TFLOPs": round(10 * d * pairs / (ms / 1000.0) / 1e12, 2),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }


def linear_bwd_cpu_baseline(inp, g_host, st_host, rule, heads_run=1):
    """The oracle's linear-branch gradient (fp64 autograd) on `heads_run`
    whole heads, scaled to the whole job's tokens/s."""
    import numpy as np
    import torch
    import oracle
    from hybrid_window_softmax_amd import inputs
    cfg = inp.cfg
    S = cfg["tokens_per_frame"]
    t0 = time.perf_counter()
    for h in range(heads_run):
        g = inputs.bf16_bits_to_f32(g_host[0, h]) if g_host.dtype == np.uint16 else g_host[0, h]
        oracle.linear_branch_grad(inp.f64("q", 0, h), inp.f64("k", 0, h), inp.f64("v", 0, h),
                                  inp.beta[0, h], inp.alpha[0, h], inp.f64("gate", 0, h),
                                  st_host[0, h], inp.conv_k[h], inp.conv_v[h], inp.rms_weight,
                                  g.astype(np.float64), S, cfg["chunk"], cfg["radius"], rule,
                                  cfg["c"], 0.5, 1e-6)
    dt = time.perf_counter() - t0
    N = cfg["frames"] * S
    total_s = dt * cfg["heads"] * cfg["batch"] / heads_run
    return {"value": N * cfg["batch"] / total_s, "unit": "tokens/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{heads_run} of {cfg['heads']} heads (all {N} tokens of each), "
                      f"{dt:.1f} s wall, scaled by heads"}


def bench_linear_bwd(args, cfg, inp, up):
    """One step = one hwa_linear_bwd over the whole workload (every input and
    the upstream gradient resident in HBM)."""
    import torch
    from hybrid_window_softmax_amd import hwa, inputs
    g_host = inputs.grad_output(cfg)
    st_host = inputs.state_matrix(cfg)
    t = {n: up(getattr(inp, n)) for n in ("q", "k", "v", "gate", "beta", "alpha", "conv_k",
                                          "conv_v", "rms_weight")}
    g = up(g_host)
    text = up(st_host)
    F, S = cfg["frames"], cfg["tokens_per_frame"]
    B, H, N, d = t["q"].shape
    grads = None

    def call(events=None, ws=None):
        nonlocal grads
        grads, ws = hwa.linear_bwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"], text,
                                   t["conv_k"], t["conv_v"], g, F, S, cfg["chunk"], cfg["radius"],
                                   args.rule, cfg["c"], 0.5, 1e-6, t["rms_weight"], grads=grads,
                                   workspace=ws, stage_events=events)
        return ws

    log("bench: linear-branch backward warmup")
    ws = call()
    for _ in range(max(0, args.warmup - 1)):
        call(ws=ws)
    torch.cuda.synchronize()
    timer = hwa.StageTimer(args.steps, hwa.NUM_LIN_BWD_STAGE_EVENTS, hwa.LIN_BWD_STAGES)
    log(f"bench: timing {args.steps} linear backward steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(events=timer.sets[i], ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage = timer.stage_ms()
    timer.close()
    ms = (t1 - t0) * 1000.0 / args.steps
    log("bench: stage ms " + ", ".join(f"{k} {v:.3f}" for k, v in stage.items()))
    io = 2 if cfg["dtype"] == "bf16" else 4
    tok = B * H * N
    # fp32 products per token: readout S_t q^, S_t^T do, do q^^T (3 x 2 d^2);
    # statistics (dA + dA^T) k^, dB k^, dB^T v^ (3 x 2 d^2)
    work = {
        "readout": dict(flops=6 * d * d * tok, bytes=0),
        "stats": dict(flops=6 * d * d * tok, bytes=0),
        # read the fp32 gradients before the convs and k, v; write dk, dv
        "convs": dict(flops=0, bytes=tok * d * (2 * 4 + 4 * io)),
    }
    kernels = {}
    for name in hwa.LIN_BWD_STAGES:
        rec = {"ms": round(stage[name], 4)}
        w = work.get(name)
        if w:
            sec = stage[name] / 1000.0
            if w["flops"]:
                rec["TFLOPs"] = round(w["flops"] / sec / 1e12, 2)
                rec["frac"] = round(w["flops"] / sec / 1e12 / PEAK_FP32_TFLOPS, 4)
            if w["bytes"]:
                rec["hbm_GBs"] = round(w["bytes"] / sec / 1e9, 1)
                rec["hbm_frac"] = round(w["bytes"] / sec / 1e9 / PEAK_HBM_GBS, 4)
        kernels[name] = rec
    dom = max(("readout", "stats"), key=lambda n: stage[n])
    achieved = work[dom]["flops"] / (stage[dom] / 1000.0) / 1e12
    # d = 64, 128: fp32 MFMA kernels (peak = the fp32 MFMA rate, the same
    # figure as the fp32 vector rate); d = 16, 32: fp32 VALU kernels. traffic:
    # the counters were taken on the 132,600-token clip only
    mfma = d in (64, 128)
    kname = f"lin_{dom}_bwd{'_mfma' if mfma else ''}_kernel"
    roofline = {"kernel": kname, "bound": "mfma" if mfma else "alu",
                "achieved": round(achieved, 2), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                "traffic": linear_bwd_traffic(kname) if cfg["name"] == "long-clip-832x480-85f"
                else None,
                "algorithmic_flops_per_launch": work[dom]["flops"]}
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle's linear-branch gradient on a sample")
        del t, g, text, grads, ws
        torch.cuda.empty_cache()
        cpu = linear_bwd_cpu_baseline(inp, g_host, st_host, args.rule, args.cpu_heads or 1)
    return {
        "metric": "linear-branch backward (dq, dk, dv, dbeta, dalpha, dgate, dS_text, dconv, "
                  "dw) tokens/s",
        "value": round(B * N / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: B{B} H{H} d{d} F{F} x S{S} = {N} tokens, "
                               f"chunk {cfg['chunk']} radius {cfg['radius']}, {args.rule}, "
                               f"{cfg['dtype']} I/O, linear branch backward",
                   "tokens": N, "heads": H, "head_dim": d},
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }


def bench_block(args, cfg, inp, up):
    """One step = one hwa_block_fwd over the workload: the QKV projection of a
    block input x [B, N, H d] (with the 3D RoPE in its epilogue), the hybrid
    attention of every head, the output projection."""
    import numpy as np
    import torch
    from hybrid_window_softmax_amd import hwa, inputs
    B, H, d = cfg["batch"], cfg["heads"], cfg["head_dim"]
    F, S = cfg["frames"], cfg["tokens_per_frame"]
    N, D = F * S, H * d
    grid_w = BLOCK_GRID_W.get(S, S)
    xb, wqb, wob = inputs.block_inputs(cfg)
    cpu = None
    if not args.no_cpu_baseline:
        # first, while no GPU state exists in this process: the pool forks
        log("bench: timing the CPU oracle on a sample")
        att = cpu_baseline(inp, args.rule, args.cpu_heads)
        ns = min(N, 2048)
        x64 = inputs.bf16_bits_to_f32(xb[0, :ns]).astype(np.float64)
        wq64 = inputs.bf16_bits_to_f32(wqb).astype(np.float64)
        wo64 = inputs.bf16_bits_to_f32(wob).astype(np.float64)
        t0 = time.perf_counter()
        x64 @ wq64.T
        x64 @ wo64.T  # the output projection has the same shape as x @ W_o^T
        dt = time.perf_counter() - t0
        proj_s = dt * (B * N) / ns
        tok = B * N
        total_s = tok / att["value"] + proj_s
        cpu = dict(att, value=tok / total_s,
                   sample=att["sample"] + f"; the two projections (fp64 numpy matmuls, BLAS "
                   f"threads) timed on {ns} tokens ({dt:.2f} s) and scaled by tokens")
    t = {n: up(getattr(inp, n)) for n in ("beta", "alpha", "gate", "conv_k", "conv_v",
                                          "rms_weight", "k_txt", "v_txt", "beta_txt")}
    text = hwa.text_state(t["k_txt"], t["v_txt"], t["beta_txt"]) if t["k_txt"] is not None \
        else None
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)  # noqa: E731
    x, wq, wo = to(xb), to(wqb), to(wob)
    y = torch.empty_like(x)

    def call(events=None, ws=None):
        return hwa.block_fwd(x, wq, wo, t["beta"], t["alpha"], t["gate"], text, t["conv_k"],
                             t["conv_v"], H, F, S, grid_w, 10000.0, cfg["chunk"], cfg["radius"],
                             args.rule, cfg["c"], 0.5, 1e-6, t["rms_weight"], y=y, workspace=ws,
                             stage_events=events)[1]

    log("bench: block warmup")
    ws = call()
    for _ in range(max(0, args.warmup - 1)):
        call(ws=ws)
    torch.cuda.synchronize()
    timer = hwa.StageTimer(args.steps, hwa.NUM_BLOCK_STAGE_EVENTS, hwa.BLOCK_STAGES)
    log(f"bench: timing {args.steps} block steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(events=timer.sets[i], ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage = timer.stage_ms()
    timer.close()
    ms = (t1 - t0) * 1000.0 / args.steps
    log("bench: stage ms " + ", ".join(f"{k} {v:.3f}" for k, v in stage.items()))
    M = B * N
    flops = {"qkv": 2 * M * D * 3 * D, "out_proj": 2 * M * D * D}
    kernels = {}
    for name in hwa.BLOCK_STAGES:
        rec = {"ms": round(stage[name], 4)}
        if name in flops:
            tf = flops[name] / (stage[name] / 1000.0) / 1e12
            rec["TFLOPs"] = round(tf, 2)
            rec["frac"] = round(tf / PEAK_BF16_TFLOPS, 4)
        kernels[name] = rec
    achieved = flops["qkv"] / (stage["qkv"] / 1000.0) / 1e12
    roofline = {"kernel": "gemm_nt_kernel (QKV projection, RoPE epilogue)", "bound": "mfma",
                "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "algorithmic_flops_per_launch": flops["qkv"]}
    return {
        "metric": "hybrid attention block (QKV projection + 3D RoPE, hybrid attention, output "
                  "projection) tokens/s",
        "value": round(B * N / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: B{B} H{H} d{d} F{F} x S{S} = {N} tokens, "
                               f"D {D}, latent grid {grid_w} wide, chunk {cfg['chunk']} radius "
                               f"{cfg['radius']}, {args.rule}, attention block",
                   "tokens": N, "heads": H, "head_dim": d},
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }


def bench_train_step(args, cfg, inp, up):
    """One step = the forward (keeping o_sm and its log-sum-exp), the softmax
    branch's backward, then the linear branch's backward adding its dq, dk, dv
    to the softmax branch's: every input's gradient of out = o_sm + y."""
    import torch
    from hybrid_window_softmax_amd import hwa, inputs
    g_host = inputs.grad_output(cfg)
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle's forward and gradients on a sample")
        g_host_st = inputs.state_matrix(cfg)
        hr = args.cpu_heads or 1
        parts = [cpu_baseline(inp, args.rule, hr),
                 softmax_bwd_cpu_baseline(inp, g_host, hr),
                 linear_bwd_cpu_baseline(inp, g_host, g_host_st, args.rule, hr)]
        tok = cfg["batch"] * cfg["frames"] * cfg["tokens_per_frame"]
        total_s = sum(tok / p["value"] for p in parts)
        cpu = {"value": tok / total_s, "unit": "tokens/s", "cores": parts[0]["cores"],
               "kind": "oracle",
               "sample": f"{hr} of {cfg['heads']} heads (all tokens of each) of the forward "
                         "(worker pool), the softmax gradient and the linear-branch gradient "
                         "(BLAS threads), each scaled by heads",
               **host_info()}
    t = {n: up(getattr(inp, n)) for n in ("q", "k", "v", "gate", "beta", "alpha", "conv_k",
                                          "conv_v", "rms_weight", "k_txt", "v_txt",
                                          "beta_txt")}
    text = hwa.text_state(t["k_txt"], t["v_txt"], t["beta_txt"]) if t["k_txt"] is not None \
        else None
    g = up(g_host)
    F, S, ch, r = cfg["frames"], cfg["tokens_per_frame"], cfg["chunk"], cfg["radius"]
    q = t["q"]
    B, H, N, d = q.shape
    out, o_sm = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    st = {"wf": None, "ws": None, "wl": None, "grads": None}

    def step(ev=None, sev=None):
        if ev:
            ev[0].record()
        _, st["wf"] = hwa.hybrid_attn_fwd(q, t["k"], t["v"], t["beta"], t["alpha"], t["gate"], text,
                                          t["conv_k"], t["conv_v"], F, S, ch, r, args.rule,
                                          cfg["c"], 0.5, 1e-6, t["rms_weight"], out=out,
                                          workspace=st["wf"], softmax_lse=lse, softmax_out=o_sm)
        if ev:
            ev[1].record()
        st["ws"] = hwa.softmax_bwd(q, t["k"], t["v"], o_sm, lse, g, F, S, ch, r, dq=dq, dk=dk,
                                   dv=dv, workspace=st["ws"], stage_events=sev)[3]
        if ev:
            ev[2].record()
        grads = dict(st["grads"] or {}, q=dq, k=dk, v=dv)
        st["grads"], st["wl"] = hwa.linear_bwd(q, t["k"], t["v"], t["beta"], t["alpha"], t["gate"],
                                               text, t["conv_k"], t["conv_v"], g, F, S, ch, r,
                                               args.rule, cfg["c"], 0.5, 1e-6, t["rms_weight"],
                                               grads=grads, workspace=st["wl"], accumulate=True)
        if ev:
            ev[3].record()

    log("bench: training step warmup")
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    timer = hwa.StageTimer(args.steps, hwa.NUM_BWD_STAGE_EVENTS, hwa.BWD_STAGES)
    log(f"bench: timing {args.steps} training steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i], timer.sets[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1000.0 / args.steps
    phases = {}
    for j, name in enumerate(("forward", "softmax_bwd", "linear_bwd")):
        phases[name] = {"ms": round(sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps, 4)}
    stage = timer.stage_ms()
    timer.close()
    log("bench: phase ms " + ", ".join(f"{k} {v['ms']:.3f}" for k, v in phases.items()))
    pairs = window_pairs(cfg) * B * H
    dkdv_flops = 8 * d * pairs
    achieved = dkdv_flops / (stage["dkdv"] / 1000.0) / 1e12
    roofline = {"kernel": "softmax_bwd_dkdv_kernel", "bound": "mfma",
                "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(BWD_TRAFFIC_FILE, SOFTMAX_BWD_SRCS)
                if cfg["name"] == "long-clip-832x480-85f" else None,
                "algorithmic_flops_per_launch": dkdv_flops}
    return {
        "metric": "hybrid attention training step (forward + backward, every input's gradient) "
                  "tokens/s",
        "value": round(B * N / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: B{B} H{H} d{d} F{F} x S{S} = {N} tokens, "
                               f"chunk {ch} radius {r}, {args.rule}, forward + backward",
                   "tokens": N, "heads": H, "head_dim": d},
        "roofline": roofline,
        "phases": phases,
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long-clip-832x480-85f",
                    help="a name in hybrid_window_softmax_amd.inputs.WORKLOADS")
    ap.add_argument("--rule", default="vdn_solve")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="heads of the CPU oracle's sample (default: two tasks per worker)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-range", action="store_true",
                    help="skip the other rules and full-size workloads of the metric's range")
    ap.add_argument("--range-steps", type=int, default=10)
    ap.add_argument("--route-tau", type=float, default=1.5,
                    help="also time the block-sparse routed softmax at this threshold "
                         "(approximate; reported under 'routed')")
    ap.add_argument("--no-routed", dest="route_tau", action="store_const", const=None)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (three times), the "
                         "reference kernel for scaling HBM byte counters")
    ap.add_argument("--train-step", action="store_true",
                    help="time forward + both backward passes (every input's gradient) instead")
    ap.add_argument("--linear-bwd", action="store_true",
                    help="time the linear branch's backward (hwa_linear_bwd) instead")
    ap.add_argument("--block", action="store_true",
                    help="time the attention block (hwa_block_fwd: projections + RoPE + hybrid "
                         "attention) instead")
    ap.add_argument("--softmax-bwd", action="store_true",
                    help="time the windowed-softmax backward (hwa_softmax_bwd) instead")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only time the vendor library's square bf16 GEMMs (torch.matmul on "
                         "hipBLASLt), the practical MFMA rate this GPU sustains, for context")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (the hot path shards by "
              "heads with no exchange; see the sharding design). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from hybrid_window_softmax_amd import hwa, inputs

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": nbytes, "copies": 3}), flush=True)
        return
    if args.gemm_ceiling:
        torch.manual_seed(0)
        for n, reps in ((8192, 20), (16384, 5)):
            a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
            b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
            for _ in range(3):
                c = a @ b
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                c = a @ b
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            print(json.dumps({"gemm": f"bf16 {n}x{n}x{n}", "ms": round(ms, 4),
                              "TFLOP/s": round(2 * n ** 3 / ms / 1e9, 1)}), flush=True)
            del a, b, c
        return

    cfg = inputs.WORKLOADS[args.workload]
    log(f"bench: generating workload {args.workload}")
    inp = inputs.make(cfg)
    dev = torch.device("cuda:0")
    bf = cfg["dtype"] == "bf16"

    def up(a):
        if a is None:
            return None
        if bf and a.dtype.name == "uint16":
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    if args.softmax_bwd:
        print(json.dumps(bench_softmax_bwd(args, cfg, inp, up)), flush=True)
        return
    if args.block:
        print(json.dumps(bench_block(args, cfg, inp, up)), flush=True)
        return
    if args.linear_bwd:
        print(json.dumps(bench_linear_bwd(args, cfg, inp, up)), flush=True)
        return
    if args.train_step:
        print(json.dumps(bench_train_step(args, cfg, inp, up)), flush=True)
        return

    cpu = None
    if not args.no_cpu_baseline:
        # first, while no GPU state exists in this process: the pool forks
        log("bench: timing the CPU oracle on a sample")
        cpu = cpu_baseline(inp, args.rule, args.cpu_heads)
    res = time_forward(cfg, inp, args.rule, args.steps, args.warmup, up)
    F, S = cfg["frames"], cfg["tokens_per_frame"]
    tokens = cfg["batch"] * F * S
    ms = res["ms"]
    routed = None
    if args.route_tau is not None:
        routed = time_routed(cfg, inp, args.rule, args.route_tau, args.range_steps, up, ms)
    rng = None
    if not args.no_range:
        # the rest of the metric's range: the other rules on this workload and
        # the other full-size workloads, each timed the same way
        rng = {}
        cases = [(cfg["name"], r) for r in cfg["rules"] if r != args.rule]
        cases += [(n, "vdn_solve") for n in RANGE_WORKLOADS if n != cfg["name"]]
        for name, rule in cases:
            c2 = inputs.WORKLOADS[name]
            log(f"bench: range entry {name} {rule}")
            inp2 = inp if name == cfg["name"] else inputs.make(c2)
            r2 = time_forward(c2, inp2, rule, args.range_steps, 2, make_up(c2))
            rng[f"{name} {rule}"] = {
                "tokens": c2["batch"] * c2["frames"] * c2["tokens_per_frame"],
                "ms_per_step": round(r2["ms"], 4),
                "tokens_per_s": round(c2["batch"] * c2["frames"] * c2["tokens_per_frame"]
                                      / (r2["ms"] / 1000.0), 1),
                "softmax_frac": r2["roofline"]["frac"],
                "hbm_frac": {k: v["hbm_frac"] for k, v in r2["kernels"].items()
                             if k != "softmax"},
            }
            del inp2
    rec = {
        "metric": "hybrid-attn fwd tokens/s at 48k-262k tokens; % of MFMA / HBM roofline",
        "value": round(tokens / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: B{cfg['batch']} H{cfg['heads']} "
                               f"d{cfg['head_dim']} F{F} x S{S} = {F * S} tokens, "
                               f"chunk {cfg['chunk']} radius {cfg['radius']}, "
                               f"{args.rule}, text state from {cfg['text_tokens']} tokens",
                   "tokens": F * S, "heads": cfg["heads"], "head_dim": cfg["head_dim"],
                   "rule": args.rule},
        "roofline": res["roofline"],
        "kernels": res["kernels"],
        "range": rng,
        "routed": routed,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def make_up(cfg):
    """Host array -> device tensor for a workload (bf16 bits become bf16)."""
    import torch
    dev = torch.device("cuda:0")
    bf = cfg["dtype"] == "bf16"

    def up(a):
        if a is None:
            return None
        if bf and a.dtype.name == "uint16":
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)
    return up


def time_routed(cfg, inp, rule, tau, steps, up, dense_ms):
    """The block-sparse routed forward (HWA_FLAG_ROUTED) on the same workload:
    time per call, the kept fraction of the window's key blocks, and the
    routed o_sm's relative Frobenius error against the dense o_sm (both from
    softmax-only calls, every head)."""
    import torch
    from hybrid_window_softmax_amd import hwa
    t = {n: up(getattr(inp, n)) for n in ("q", "k", "v", "gate", "beta", "alpha", "conv_k",
                                          "conv_v", "rms_weight", "k_txt", "v_txt",
                                          "beta_txt")}
    text = hwa.text_state(t["k_txt"], t["v_txt"], t["beta_txt"]) if t["k_txt"] is not None \
        else None
    out = torch.empty_like(t["q"])
    F, S = cfg["frames"], cfg["tokens_per_frame"]

    def call(tau_, flags=0, ws=None, o=out, events=None):
        return hwa.hybrid_attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"],
                                   text, t["conv_k"], t["conv_v"], F, S, cfg["chunk"],
                                   cfg["radius"], rule, cfg["c"], 0.5, 1e-6, t["rms_weight"],
                                   flags=flags, out=o, workspace=ws, route_tau=tau_,
                                   stage_events=events)[1]

    log(f"bench: routed softmax, tau {tau}")
    ws = call(tau)
    for _ in range(2):
        call(tau, ws=ws)
    torch.cuda.synchronize()
    timer = hwa.StageTimer(steps)
    t0 = time.perf_counter()
    for i in range(steps):
        call(tau, ws=ws, events=timer.sets[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    stage = timer.stage_ms()
    timer.close()
    B, H = cfg["batch"], cfg["heads"]
    p = hwa.make_params(B, H, cfg["head_dim"], torch.bfloat16, flags=hwa.FLAG_ROUTED)
    L = hwa.route_layout(F, S, cfg["chunk"], p)
    nch = -(-F // cfg["chunk"])
    tpc = L["tiles_per_chunk"]
    cnt = ws[L["count"]:L["count"] + B * H * nch * tpc * 4].view(torch.int32).view(
        B * H, nch, tpc).to(torch.float64)
    # blocks of each chunk's window (every tile of a chunk sees the same window)
    lo, hi = [], []
    for c in range(nch):
        f0 = c * cfg["chunk"]
        lo.append(max(0, (c - cfg["radius"]) * cfg["chunk"]) * S)
        hi.append((min(F - 1, (c + cfg["radius"] + 1) * cfg["chunk"] - 1) + 1) * S)
        del f0
    nkb = torch.tensor([(h_ - 1) // 128 - l_ // 128 + 1 for l_, h_ in zip(lo, hi)],
                       dtype=torch.float64, device=cnt.device)
    ntq = torch.tensor([-(-(min(F, (c + 1) * cfg["chunk"]) - c * cfg["chunk"]) * S // 256)
                        for c in range(nch)], device=cnt.device)
    valid = torch.arange(tpc, device=cnt.device)[None, :] < ntq[:, None]
    kept = float((cnt * valid).sum())
    total = float((valid * nkb[:, None]).sum() * B * H)
    dense_sm = torch.empty_like(out)
    routed_sm = torch.empty_like(out)
    call(None, hwa.FLAG_SOFTMAX_ONLY, None, dense_sm)
    call(tau, hwa.FLAG_SOFTMAX_ONLY, ws, routed_sm)
    torch.cuda.synchronize()
    a = routed_sm.float().view(B * H, -1)
    r = dense_sm.float().view(B * H, -1)
    err = float(((a - r).norm(dim=1) / r.norm(dim=1)).max())
    del t, text, out, ws, dense_sm, routed_sm, a, r
    torch.cuda.empty_cache()
    return {"tau": tau, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(B * F * S / (ms / 1000.0), 1),
            "speedup_vs_dense": round(dense_ms / ms, 3),
            "softmax_ms": round(stage["softmax"], 4),
            "routing_and_vtranspose_ms": round(stage["vtranspose"], 4),
            "kept_block_fraction": round(kept / total, 4),
            "o_sm_rel_err_vs_dense": round(err, 4)}


def time_forward(cfg, inp, rule, steps, warmup, up):
    """Time `steps` hybrid_attn_fwd calls on a workload (after `warmup`
    untimed ones): wall time per call, every stage's hipEvent time and rates,
    and the softmax kernel's roofline. Frees its device memory."""
    import torch
    from hybrid_window_softmax_amd import hwa
    t = {n: up(getattr(inp, n)) for n in ("q", "k", "v", "gate", "beta", "alpha", "conv_k",
                                          "conv_v", "rms_weight", "k_txt", "v_txt",
                                          "beta_txt")}
    text = None
    if t["k_txt"] is not None:
        text = hwa.text_state(t["k_txt"], t["v_txt"], t["beta_txt"])
    out = torch.empty_like(t["q"])
    F, S = cfg["frames"], cfg["tokens_per_frame"]

    def call(events=None, ws=None):
        return hwa.hybrid_attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["gate"],
                                   text, t["conv_k"], t["conv_v"], F, S, cfg["chunk"],
                                   cfg["radius"], rule, cfg["c"], 0.5, 1e-6,
                                   t["rms_weight"], out=out, workspace=ws,
                                   stage_events=events)[1]

    log(f"bench: {cfg['name']} {rule}: warmup")
    ws = call()
    for _ in range(max(0, warmup - 1)):
        call(ws=ws)
    torch.cuda.synchronize()
    timer = hwa.StageTimer(steps)
    log(f"bench: {cfg['name']} {rule}: timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(events=timer.sets[i], ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage = timer.stage_ms()
    timer.close()
    ms = (t1 - t0) * 1000.0 / steps
    log("bench: stage ms " + ", ".join(f"{k} {v:.3f}" for k, v in stage.items()))

    bf = cfg["dtype"] == "bf16"
    work = algorithmic_work(cfg)
    fused = bf  # the library fuses the readout into the softmax on bf16 (no q_rope)
    if fused:
        work["softmax"] = work.pop("softmax+readout")
        work.pop("readout")
    else:
        work.pop("softmax+readout")
    if bf and cfg["tokens_per_frame"] % 4 == 0:
        # the statistics kernel writes the softmax's transposed v itself
        vt = work.pop("vtranspose")
        work["stats"]["bytes"] += vt["bytes"] // 2
    kernels = {}
    for name, w in work.items():
        sec = stage[name] / 1000.0
        if sec <= 0:
            continue
        rec = {"ms": round(stage[name], 4),
               "hbm_GBs": round(w["bytes"] / sec / 1e9, 1),
               "hbm_frac": round(w["bytes"] / sec / 1e9 / PEAK_HBM_GBS, 4)}
        if w["flops"]:
            rec["TFLOPs"] = round(w["flops"] / sec / 1e12, 2)
        kernels[name] = rec
    sm_flops = work["softmax"]["flops"]
    achieved = sm_flops / (stage["softmax"] / 1000.0) / 1e12
    roofline = {"kernel": "softmax_bf16_kernel" + (" (readout fused)" if fused else ""),
                "bound": "mfma",
                "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": softmax_traffic() if cfg["name"] == TRAFFIC_WORKLOAD else None,
                "algorithmic_flops_per_launch": sm_flops}
    del t, text, out, ws
    torch.cuda.empty_cache()
    return {"ms": ms, "stage": stage, "kernels": kernels, "roofline": roofline}


if __name__ == "__main__":
    main()
