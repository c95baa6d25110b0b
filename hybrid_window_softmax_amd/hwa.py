"""ctypes binding of libhwa.so (include/hwa.h).

Argument marshalling only: every step of the hybrid attention runs in the HIP
kernels behind the C ABI. PyTorch supplies device memory and the stream. The
library must have been built (``python -m hybrid_window_softmax_amd.build``);
there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhwa.so")
_lib = None

RULES = {"vdn_solve": 0, "sana_scaled": 1, "vdn_scaled": 2}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
FLAG_SOFTMAX_ONLY = 1
FLAG_LINEAR_ONLY = 2
FLAG_ACCUMULATE = 8
FLAG_ROUTED = 16
NUM_STAGE_EVENTS = 9
STAGES = ("window", "stats", "inverse", "scan", "decay+state", "vtranspose", "softmax",
          "readout")
NUM_BWD_STAGE_EVENTS = 4
BWD_STAGES = ("prep", "dq", "dkdv")
NUM_LIN_BWD_STAGE_EVENTS = 6
NUM_BLOCK_STAGE_EVENTS = 4
BLOCK_STAGES = ("qkv", "attention", "out_proj")
LIN_BWD_STAGES = ("recompute", "readout", "scans", "stats", "convs")
# gradients hwa_linear_bwd returns, in its argument order
LIN_GRADS = ("q", "k", "v", "beta", "alpha", "gate", "text_state", "conv_k", "conv_v",
             "rms_weight")

HWA_OK = 0
HWA_ERR_INVALID_ARG = 1
HWA_ERR_UNSUPPORTED = 2
HWA_ERR_WORKSPACE = 3
HWA_ERR_HIP = 4
HWA_F32 = 0
HWA_BF16 = 1

EXPORTS = ("hybrid_attn_fwd", "hybrid_attn_fwd_noalloc", "hwa_workspace_bytes", "hwa_get_workspace_layout",
           "hwa_window_bounds", "hwa_text_state", "hwa_text_state_workspace_bytes",
           "hwa_softmax_bwd", "hwa_softmax_bwd_workspace_bytes", "hwa_linear_bwd",
           "hwa_linear_bwd_workspace_bytes", "hwa_frame_alpha", "hwa_block_fwd",
           "hwa_block_workspace_bytes", "hwa_get_route_layout", "hwa_status_string")


class Params(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("c", ctypes.c_float),
        ("text_scale", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("conv_k", ctypes.c_void_p),
        ("conv_v", ctypes.c_void_p),
        ("rms_weight", ctypes.c_void_p),
        ("q_rope", ctypes.c_void_p),
        ("k_rope", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("flags", ctypes.c_uint32),
        ("stage_events", ctypes.c_void_p),
        ("softmax_lse", ctypes.c_void_p),
        ("softmax_out", ctypes.c_void_p),
        ("route_tau", ctypes.c_float),
    ]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("lohi", "stat_a", "stat_b", "map_m", "bank_p", "bank_q", "decay",
                 "bank_e", "v_t", "st16", "st_eps", "total")]


class HwaError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__(lib().hwa_status_string(code).decode())


def lib():
    """Load libhwa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m hybrid_window_softmax_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        PP = ctypes.POINTER(Params)
        L.hybrid_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                      i32, vp, vp, PP]
        L.hybrid_attn_fwd.restype = ctypes.c_int
        L.hybrid_attn_fwd_noalloc.argtypes = L.hybrid_attn_fwd.argtypes
        L.hybrid_attn_fwd_noalloc.restype = ctypes.c_int
        L.hwa_workspace_bytes.argtypes = [i32, i32, i32, PP]
        L.hwa_workspace_bytes.restype = sz
        L.hwa_get_workspace_layout.argtypes = [i32, i32, i32, PP, ctypes.POINTER(Layout)]
        L.hwa_get_workspace_layout.restype = ctypes.c_int
        L.hwa_window_bounds.argtypes = [i32, i32, i32, ctypes.POINTER(i32),
                                        ctypes.POINTER(i32)]
        L.hwa_window_bounds.restype = ctypes.c_int
        L.hwa_text_state.argtypes = [vp, vp, vp, i32, vp, vp, PP]
        L.hwa_text_state.restype = ctypes.c_int
        L.hwa_text_state_workspace_bytes.argtypes = [i32, PP]
        L.hwa_text_state_workspace_bytes.restype = sz
        L.hwa_softmax_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp,
                                      vp, vp, PP]
        L.hwa_softmax_bwd.restype = ctypes.c_int
        L.hwa_softmax_bwd_workspace_bytes.argtypes = [i32, i32, i32, PP]
        L.hwa_softmax_bwd_workspace_bytes.restype = sz
        L.hwa_linear_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, PP]
        L.hwa_linear_bwd.restype = ctypes.c_int
        L.hwa_linear_bwd_workspace_bytes.argtypes = [i32, i32, i32, PP]
        L.hwa_linear_bwd_workspace_bytes.restype = sz
        L.hwa_frame_alpha.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, PP]
        L.hwa_frame_alpha.restype = ctypes.c_int
        L.hwa_block_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_float,
                                    i32, i32, i32, vp, vp, PP]
        L.hwa_block_fwd.restype = ctypes.c_int
        L.hwa_block_workspace_bytes.argtypes = [i32, i32, i32, PP]
        L.hwa_block_workspace_bytes.restype = sz
        L.hwa_get_route_layout.argtypes = [i32, i32, i32, PP, ctypes.POINTER(sz),
                                           ctypes.POINTER(sz), ctypes.POINTER(i32),
                                           ctypes.POINTER(i32)]
        L.hwa_get_route_layout.restype = ctypes.c_int
        L.hwa_status_string.argtypes = [ctypes.c_int]
        L.hwa_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_params(batch, heads, head_dim, dtype, c=0.5, text_scale=0.5,
                rms_eps=1e-6, conv_k=None, conv_v=None, rms_weight=None,
                q_rope=None, k_rope=None, workspace=None, flags=0) -> Params:
    p = Params()
    p.struct_size = ctypes.sizeof(Params)
    p.batch, p.heads, p.head_dim = batch, heads, head_dim
    p.dtype = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    p.c, p.text_scale, p.rms_eps = c, text_scale, rms_eps
    for name, t in (("conv_k", conv_k), ("conv_v", conv_v), ("rms_weight", rms_weight),
                    ("q_rope", q_rope), ("k_rope", k_rope)):
        setattr(p, name, None if t is None else t.data_ptr())
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    p.flags = flags
    return p


def window_bounds(frames: int, chunk: int, radius: int):
    """Host window table from the library (int32 lists lo, hi)."""
    lo = (ctypes.c_int32 * frames)()
    hi = (ctypes.c_int32 * frames)()
    code = lib().hwa_window_bounds(frames, chunk, radius, lo, hi)
    if code != HWA_OK:
        raise HwaError(code)
    return list(lo), list(hi)


def workspace_bytes(frames, tokens_per_frame, chunk, p: Params) -> int:
    return int(lib().hwa_workspace_bytes(frames, tokens_per_frame, chunk, ctypes.byref(p)))


def workspace_layout(frames, tokens_per_frame, chunk, p: Params) -> dict:
    L = Layout()
    code = lib().hwa_get_workspace_layout(frames, tokens_per_frame, chunk, ctypes.byref(p),
                                          ctypes.byref(L))
    if code != HWA_OK:
        raise HwaError(code)
    return {n: getattr(L, n) for n, _ in Layout._fields_}


def route_layout(frames, tokens_per_frame, chunk, p: Params) -> dict:
    """Where the routed softmax's kept-block lists sit in the workspace."""
    co, lo = ctypes.c_size_t(), ctypes.c_size_t()
    tpc, stride = ctypes.c_int32(), ctypes.c_int32()
    code = lib().hwa_get_route_layout(frames, tokens_per_frame, chunk, ctypes.byref(p),
                                      ctypes.byref(co), ctypes.byref(lo), ctypes.byref(tpc),
                                      ctypes.byref(stride))
    if code != HWA_OK:
        raise HwaError(code)
    return {"count": co.value, "list": lo.value, "tiles_per_chunk": tpc.value,
            "stride": stride.value}


def _check(t, name, dtype, shape, device):
    if t is None:
        return
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def hybrid_attn_fwd(q, k, v, beta, alpha, gate, text_state, conv_k, conv_v,
                    frames: int, tokens_per_frame: int, chunk: int = 5,
                    radius: int = 1, rule: str = "vdn_solve", c: float = 0.5,
                    text_scale: float = 0.5, rms_eps: float = 1e-6,
                    rms_weight=None, q_rope=None, k_rope=None, flags: int = 0,
                    out=None, workspace=None, stream=None, stage_events=None,
                    softmax_lse=None, softmax_out=None, noalloc=False, route_tau=None):
    """out = windowed softmax + delta-rule linear branch (see include/hwa.h).

    ``route_tau``: run the softmax branch block-sparse (FLAG_ROUTED) with this
    keep threshold (-inf keeps every block).

    ``noalloc``: call hybrid_attn_fwd_noalloc instead, which uses the
    library's own fixed scratch array (HWA_NOALLOC_SCRATCH_BYTES per GPU) and
    allocates nothing; no workspace is allocated here either (the returned
    workspace is None).

    q, k, v, gate: [B, H, N, d] bf16 or fp32 CUDA tensors; beta [B, H, N],
    alpha [B, H, F, d], text_state [B, H, d, d] (or None), conv_k/conv_v
    [H, d, 4], rms_weight [d] (or None): fp32. ``stage_events``: optional
    ctypes array of NUM_STAGE_EVENTS hipEvent_t (see :class:`StageTimer`).
    ``softmax_lse`` ([B, H, N] fp32) and ``softmax_out`` (like q), when
    given, receive the softmax branch's log-sum-exp and output.
    Returns (out, workspace).
    """
    B, H, N, d = q.shape
    dev = q.device
    _check(q, "q", q.dtype, (B, H, N, d), dev)
    for name, t in (("k", k), ("v", v), ("gate", gate), ("q_rope", q_rope),
                    ("k_rope", k_rope)):
        _check(t, name, q.dtype, (B, H, N, d), dev)
    _check(beta, "beta", torch.float32, (B, H, N), dev)
    _check(alpha, "alpha", torch.float32, (B, H, frames, d), dev)
    _check(text_state, "text_state", torch.float32, (B, H, d, d), dev)
    _check(conv_k, "conv_k", torch.float32, (H, d, 4), dev)
    _check(conv_v, "conv_v", torch.float32, (H, d, 4), dev)
    _check(rms_weight, "rms_weight", torch.float32, (d,), dev)
    _check(softmax_lse, "softmax_lse", torch.float32, (B, H, N), dev)
    _check(softmax_out, "softmax_out", q.dtype, (B, H, N, d), dev)
    if route_tau is not None:
        flags |= FLAG_ROUTED
    p = make_params(B, H, d, q.dtype, c, text_scale, rms_eps, conv_k, conv_v, rms_weight,
                    q_rope, k_rope, None, flags)
    if route_tau is not None:
        p.route_tau = route_tau
    p.softmax_lse = None if softmax_lse is None else softmax_lse.data_ptr()
    p.softmax_out = None if softmax_out is None else softmax_out.data_ptr()
    if noalloc:
        workspace = None
    else:
        need = workspace_bytes(frames, tokens_per_frame, chunk, p)
        if workspace is None:
            workspace = alloc_workspace(need, dev)
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    if stage_events is not None:
        p.stage_events = ctypes.cast(stage_events, ctypes.c_void_p)
    if out is None:
        out = torch.empty_like(q)
    st = _stream(dev) if stream is None else ctypes.c_void_p(stream)
    fn = lib().hybrid_attn_fwd_noalloc if noalloc else lib().hybrid_attn_fwd
    code = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(gate), _ptr(text_state),
              frames, tokens_per_frame, chunk, radius,
              RULES[rule] if isinstance(rule, str) else rule, _ptr(out), st, ctypes.byref(p))
    if code != HWA_OK:
        raise HwaError(code)
    return out, workspace


def softmax_bwd(q, k, v, o_sm, lse, d_o, frames: int, tokens_per_frame: int,
                chunk: int = 5, radius: int = 1, dq=None, dk=None, dv=None,
                workspace=None, stream=None, stage_events=None):
    """(dq, dk, dv) of the windowed softmax branch (hwa_softmax_bwd).

    q, k, v, o_sm, d_o: [B, H, N, d] bf16 or fp32 CUDA tensors (o_sm and lse
    from a forward call with ``softmax_out`` / ``softmax_lse``, or with
    FLAG_SOFTMAX_ONLY); lse [B, H, N] fp32. ``stage_events``: optional ctypes
    array of NUM_BWD_STAGE_EVENTS hipEvent_t. Returns (dq, dk, dv, workspace).
    """
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o_sm", o_sm), ("d_o", d_o),
                    ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, name, q.dtype, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    p = make_params(B, H, d, q.dtype)
    need = int(lib().hwa_softmax_bwd_workspace_bytes(frames, tokens_per_frame, chunk,
                                                     ctypes.byref(p)))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    p.workspace = workspace.data_ptr()
    p.workspace_bytes = workspace.numel() * workspace.element_size()
    if stage_events is not None:
        p.stage_events = ctypes.cast(stage_events, ctypes.c_void_p)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    st = _stream(dev) if stream is None else ctypes.c_void_p(stream)
    code = lib().hwa_softmax_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o_sm), _ptr(lse), _ptr(d_o),
                                 frames, tokens_per_frame, chunk, radius, _ptr(dq), _ptr(dk),
                                 _ptr(dv), st, ctypes.byref(p))
    if code != HWA_OK:
        raise HwaError(code)
    return dq, dk, dv, workspace


def linear_bwd(q, k, v, beta, alpha, gate, text_state, conv_k, conv_v, d_o, frames: int,
               tokens_per_frame: int, chunk: int = 5, radius: int = 1, rule="vdn_solve",
               c: float = 0.5, text_scale: float = 0.5, rms_eps: float = 1e-6,
               rms_weight=None, grads=None, workspace=None, stream=None,
               stage_events=None, accumulate=False):
    """Gradients of the linear branch (hwa_linear_bwd) for upstream gradient
    d_o, as a dict keyed by LIN_GRADS (``text_state`` and ``rms_weight``
    always present: at the zero state / for unit weights when not given).

    Tensors as for hybrid_attn_fwd, d_o like q. ``grads``: optional dict of
    preallocated outputs. ``stage_events``: optional ctypes array of
    NUM_LIN_BWD_STAGE_EVENTS hipEvent_t. ``accumulate``: add dq, dk, dv to
    the tensors given in ``grads`` (FLAG_ACCUMULATE). Returns (grads, workspace).
    """
    B, H, N, d = q.shape
    F = frames
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("d_o", d_o)):
        _check(t, name, q.dtype, (B, H, N, d), dev)
    _check(beta, "beta", torch.float32, (B, H, N), dev)
    _check(alpha, "alpha", torch.float32, (B, H, F, d), dev)
    _check(text_state, "text_state", torch.float32, (B, H, d, d), dev)
    _check(conv_k, "conv_k", torch.float32, (H, d, 4), dev)
    _check(conv_v, "conv_v", torch.float32, (H, d, 4), dev)
    _check(rms_weight, "rms_weight", torch.float32, (d,), dev)
    p = make_params(B, H, d, q.dtype, c, text_scale, rms_eps, conv_k, conv_v, rms_weight,
                    flags=FLAG_ACCUMULATE if accumulate else 0)
    if accumulate and any((grads or {}).get(n) is None for n in ("q", "k", "v")):
        raise ValueError("accumulate needs dq, dk and dv in grads")
    need = int(lib().hwa_linear_bwd_workspace_bytes(frames, tokens_per_frame, chunk,
                                                    ctypes.byref(p)))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    p.workspace = workspace.data_ptr()
    p.workspace_bytes = workspace.numel() * workspace.element_size()
    if stage_events is not None:
        p.stage_events = ctypes.cast(stage_events, ctypes.c_void_p)
    shapes = dict(q=(q.dtype, (B, H, N, d)), k=(q.dtype, (B, H, N, d)),
                  v=(q.dtype, (B, H, N, d)), gate=(q.dtype, (B, H, N, d)),
                  beta=(torch.float32, (B, H, N)), alpha=(torch.float32, (B, H, F, d)),
                  text_state=(torch.float32, (B, H, d, d)),
                  conv_k=(torch.float32, (H, d, 4)), conv_v=(torch.float32, (H, d, 4)),
                  rms_weight=(torch.float32, (d,)))
    g = dict(grads or {})
    for name, (dt, shp) in shapes.items():
        if g.get(name) is None:
            g[name] = torch.empty(shp, dtype=dt, device=dev)
        _check(g[name], "d" + name, dt, shp, dev)
    st = _stream(dev) if stream is None else ctypes.c_void_p(stream)
    code = lib().hwa_linear_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(gate), _ptr(text_state),
        _ptr(d_o), frames, tokens_per_frame, chunk, radius,
        RULES[rule] if isinstance(rule, str) else rule, _ptr(g["q"]), _ptr(g["k"]),
        _ptr(g["v"]), _ptr(g["beta"]), _ptr(g["alpha"]), _ptr(g["gate"]),
        _ptr(g["text_state"]), _ptr(g["conv_k"]), _ptr(g["conv_v"]), _ptr(g["rms_weight"]),
        st, ctypes.byref(p))
    if code != HWA_OK:
        raise HwaError(code)
    return g, workspace


class WindowedSoftmaxAttention(torch.autograd.Function):
    """The windowed softmax branch as an autograd function: the forward runs
    hybrid_attn_fwd with FLAG_SOFTMAX_ONLY (saving o_sm and its log-sum-exp),
    the backward runs hwa_softmax_bwd. Marshalling only: both passes are the
    library's kernels."""

    @staticmethod
    def forward(ctx, q, k, v, frames, tokens_per_frame, chunk, radius):
        B, H, N, d = q.shape
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        o, _ = hybrid_attn_fwd(q, k, v, None, None, None, None, None, None, frames,
                               tokens_per_frame, chunk, radius, flags=FLAG_SOFTMAX_ONLY,
                               softmax_lse=lse)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.geom = (frames, tokens_per_frame, chunk, radius)
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv, _ = softmax_bwd(q, k, v, o, lse, d_o.contiguous(), *ctx.geom)
        return dq, dk, dv, None, None, None, None


class HybridAttention(torch.autograd.Function):
    """out = o_sm + y of the hybrid attention as an autograd function: the
    forward is hybrid_attn_fwd (also saving o_sm and its log-sum-exp), the
    backward is hwa_softmax_bwd for dq, dk, dv of the softmax branch and then
    hwa_linear_bwd with FLAG_ACCUMULATE, which adds the linear branch's dq,
    dk, dv and writes the gradients of every other input. Marshalling only."""

    @staticmethod
    def forward(ctx, q, k, v, beta, alpha, gate, text_state, conv_k, conv_v, rms_weight,
                frames, tokens_per_frame, chunk, radius, rule, c, text_scale, rms_eps):
        B, H, N, d = q.shape
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        o_sm = torch.empty_like(q)
        out, _ = hybrid_attn_fwd(q, k, v, beta, alpha, gate, text_state, conv_k, conv_v,
                                 frames, tokens_per_frame, chunk, radius, rule, c, text_scale,
                                 rms_eps, rms_weight, softmax_lse=lse, softmax_out=o_sm)
        ctx.save_for_backward(q, k, v, beta, alpha, gate, text_state, conv_k, conv_v,
                              rms_weight, o_sm, lse)
        ctx.geom = (frames, tokens_per_frame, chunk, radius, rule, c, text_scale, rms_eps)
        ctx.has_text = text_state is not None
        ctx.has_w = rms_weight is not None
        return out

    @staticmethod
    def backward(ctx, d_out):
        (q, k, v, beta, alpha, gate, text_state, conv_k, conv_v, rms_weight, o_sm,
         lse) = ctx.saved_tensors
        F, S, chunk, radius, rule, c, text_scale, rms_eps = ctx.geom
        d_out = d_out.contiguous()
        dq, dk, dv, _ = softmax_bwd(q, k, v, o_sm, lse, d_out, F, S, chunk, radius)
        g, _ = linear_bwd(q, k, v, beta, alpha, gate, text_state, conv_k, conv_v, d_out, F, S,
                          chunk, radius, rule, c, text_scale, rms_eps, rms_weight,
                          grads=dict(q=dq, k=dk, v=dv), accumulate=True)
        return (g["q"], g["k"], g["v"], g["beta"], g["alpha"], g["gate"],
                g["text_state"] if ctx.has_text else None, g["conv_k"], g["conv_v"],
                g["rms_weight"] if ctx.has_w else None,
                None, None, None, None, None, None, None, None)


def hybrid_attention(q, k, v, beta, alpha, gate, text_state, conv_k, conv_v, frames: int,
                     tokens_per_frame: int, chunk: int = 5, radius: int = 1,
                     rule="vdn_solve", c: float = 0.5, text_scale: float = 0.5,
                     rms_eps: float = 1e-6, rms_weight=None):
    """out = o_sm + y, differentiable in every tensor input (all three update
    rules, sana_scaled within the range hwa_linear_bwd states; no q_rope /
    k_rope)."""
    return HybridAttention.apply(q, k, v, beta, alpha, gate, text_state, conv_k, conv_v,
                                 rms_weight, frames, tokens_per_frame, chunk, radius, rule, c,
                                 text_scale, rms_eps)


def windowed_softmax_attention(q, k, v, frames: int, tokens_per_frame: int, chunk: int = 5,
                               radius: int = 1):
    """o_sm of the windowed softmax branch, differentiable in q, k and v."""
    return WindowedSoftmaxAttention.apply(q, k, v, frames, tokens_per_frame, chunk, radius)


def text_state(k_txt, v_txt, beta_txt, workspace=None, out=None):
    """S_text [B, H, d, d] fp32 from text tokens (hwa_text_state)."""
    B, H, T, d = k_txt.shape
    dev = k_txt.device
    _check(v_txt, "v_txt", k_txt.dtype, (B, H, T, d), dev)
    _check(beta_txt, "beta_txt", torch.float32, (B, H, T), dev)
    p = make_params(B, H, d, k_txt.dtype)
    need = int(lib().hwa_text_state_workspace_bytes(T, ctypes.byref(p)))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    p.workspace = workspace.data_ptr()
    p.workspace_bytes = workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    code = lib().hwa_text_state(_ptr(k_txt), _ptr(v_txt), _ptr(beta_txt), T, _ptr(out),
                                _stream(dev), ctypes.byref(p))
    if code != HWA_OK:
        raise HwaError(code)
    return out


def frame_alpha(k, w, bias, a_log, frames: int, tokens_per_frame: int, out=None,
                stream=None):
    """alpha [B, H, F, d] fp32 = exp(-exp(a_log) softplus(mean_frame(k) w + bias))
    (hwa_frame_alpha). k: [B, H, N, d] bf16 or fp32; w: [H, d, d]; bias,
    a_log: [H, d] fp32."""
    B, H, N, d = k.shape
    dev = k.device
    _check(k, "k", k.dtype, (B, H, N, d), dev)
    _check(w, "w", torch.float32, (H, d, d), dev)
    _check(bias, "bias", torch.float32, (H, d), dev)
    _check(a_log, "a_log", torch.float32, (H, d), dev)
    if out is None:
        out = torch.empty((B, H, frames, d), dtype=torch.float32, device=dev)
    _check(out, "alpha", torch.float32, (B, H, frames, d), dev)
    p = make_params(B, H, d, k.dtype)
    st = _stream(dev) if stream is None else ctypes.c_void_p(stream)
    code = lib().hwa_frame_alpha(_ptr(k), _ptr(w), _ptr(bias), _ptr(a_log), frames,
                                 tokens_per_frame, _ptr(out), st, ctypes.byref(p))
    if code != HWA_OK:
        raise HwaError(code)
    return out


def block_fwd(x, w_qkv, w_o, beta, alpha, gate, text_state, conv_k, conv_v, heads: int,
              frames: int, tokens_per_frame: int, grid_w: int, rope_theta: float = 10000.0,
              chunk: int = 5, radius: int = 1, rule="vdn_solve", c: float = 0.5,
              text_scale: float = 0.5, rms_eps: float = 1e-6, rms_weight=None, y=None,
              workspace=None, stream=None, stage_events=None):
    """The attention block (hwa_block_fwd): y = concat_h(hybrid attention of
    the projected, 3D-rotated heads) W_o^T. x [B, N, D] bf16 with D = heads *
    d; w_qkv [3 D, D], w_o [D, D] bf16; beta [B, H, N], alpha [B, H, F, d],
    gate [B, H, N, d] (bf16), text_state [B, H, d, d] or None, conv taps
    [H, d, 4], rms_weight [d] or None. Returns (y, workspace)."""
    B, N, D = x.shape
    H = heads
    d = D // H
    dev = x.device
    _check(x, "x", torch.bfloat16, (B, N, D), dev)
    _check(w_qkv, "w_qkv", torch.bfloat16, (3 * D, D), dev)
    _check(w_o, "w_o", torch.bfloat16, (D, D), dev)
    _check(beta, "beta", torch.float32, (B, H, N), dev)
    _check(alpha, "alpha", torch.float32, (B, H, frames, d), dev)
    _check(gate, "gate", torch.bfloat16, (B, H, N, d), dev)
    _check(text_state, "text_state", torch.float32, (B, H, d, d), dev)
    _check(conv_k, "conv_k", torch.float32, (H, d, 4), dev)
    _check(conv_v, "conv_v", torch.float32, (H, d, 4), dev)
    _check(rms_weight, "rms_weight", torch.float32, (d,), dev)
    p = make_params(B, H, d, torch.bfloat16, c, text_scale, rms_eps, conv_k, conv_v, rms_weight)
    need = int(lib().hwa_block_workspace_bytes(frames, tokens_per_frame, chunk, ctypes.byref(p)))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    p.workspace = workspace.data_ptr()
    p.workspace_bytes = workspace.numel() * workspace.element_size()
    if stage_events is not None:
        p.stage_events = ctypes.cast(stage_events, ctypes.c_void_p)
    if y is None:
        y = torch.empty_like(x)
    st = _stream(dev) if stream is None else ctypes.c_void_p(stream)
    code = lib().hwa_block_fwd(_ptr(x), _ptr(w_qkv), _ptr(w_o), _ptr(beta), _ptr(alpha),
                               _ptr(gate), _ptr(text_state), frames, tokens_per_frame, grid_w,
                               rope_theta, chunk, radius,
                               RULES[rule] if isinstance(rule, str) else rule, _ptr(y), st,
                               ctypes.byref(p))
    if code != HWA_OK:
        raise HwaError(code)
    return y, workspace


class StageTimer:
    """hipEvents recorded by the library at its kernel boundaries on the
    call's stream (hwa_params.stage_events); yields per-kernel durations."""

    def __init__(self, steps: int, n_events: int = NUM_STAGE_EVENTS, names=STAGES):
        self.n_events, self.names = n_events, names
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.sets = []
        for _ in range(steps):
            arr = (ctypes.c_void_p * self.n_events)()
            for i in range(self.n_events):
                ev = ctypes.c_void_p()
                if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = ev
            self.sets.append(arr)

    def stage_ms(self) -> dict:
        """Mean duration (ms) of every stage over the recorded steps; call
        after the stream has been synchronised."""
        tot = [0.0] * (self.n_events - 1)
        ms = ctypes.c_float()
        for arr in self.sets:
            for i in range(self.n_events - 1):
                if self.hip.hipEventElapsedTime(ctypes.byref(ms), arr[i], arr[i + 1]) != 0:
                    raise RuntimeError("hipEventElapsedTime failed")
                tot[i] += ms.value
        return {s: t / len(self.sets) for s, t in zip(self.names, tot)}

    def close(self):
        for arr in self.sets:
            for i in range(self.n_events):
                self.hip.hipEventDestroy(arr[i])
        self.sets = []
