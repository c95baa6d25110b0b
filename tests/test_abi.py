"""C-ABI contract of libhwa on the host (no GPU needed): the library loads,
exports every entry point include/hwa.h declares, computes the window table
bit-exactly, and rejects bad arguments with the documented status before
anything is enqueued (none of these calls reaches a kernel launch)."""

import ctypes
import os
import re

import pytest
import torch

import oracle
from hybrid_window_softmax_amd import hwa, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "hwa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(hwa_[a-z_]+|hybrid_attn_fwd[a-z_]*)\s*\(", src))


def test_exports_every_declared_symbol():
    L = hwa.lib()
    names = _declared()
    assert names == set(hwa.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in range(5):
        assert hwa.lib().hwa_status_string(code).decode().startswith("HWA_")


@pytest.mark.parametrize("F", range(1, 41))
def test_window_bounds_bit_exact(F):
    for chunk in range(1, 8):
        for radius in range(0, 4):
            lo, hi = hwa.window_bounds(F, chunk, radius)
            olo, ohi = oracle.window_bounds(F, chunk, radius)
            assert lo == olo.tolist() and hi == ohi.tolist()


def test_window_bounds_workloads():
    for cfg in inputs.WORKLOADS.values():
        lo, hi = hwa.window_bounds(cfg["frames"], cfg["chunk"], cfg["radius"])
        olo, ohi = oracle.window_bounds(cfg["frames"], cfg["chunk"], cfg["radius"])
        assert lo == olo.tolist() and hi == ohi.tolist()


def test_window_bounds_bad_args():
    L = hwa.lib()
    a = (ctypes.c_int32 * 4)()
    assert L.hwa_window_bounds(0, 5, 1, a, a) == hwa.HWA_ERR_INVALID_ARG
    assert L.hwa_window_bounds(4, 0, 1, a, a) == hwa.HWA_ERR_INVALID_ARG
    assert L.hwa_window_bounds(4, 5, -1, a, a) == hwa.HWA_ERR_INVALID_ARG
    assert L.hwa_window_bounds(4, 5, 1, None, a) == hwa.HWA_ERR_INVALID_ARG


# Fake, never-dereferenced device addresses: every call below must fail
# validation on the host. They are passed only where no GPU is visible, so a
# validation bug can never turn one of them into a kernel launch.
BASE = 1 << 40
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="fake device addresses are passed only without a GPU")


def _params(**kw):
    p = hwa.make_params(kw.pop("batch", 1), kw.pop("heads", 2), kw.pop("head_dim", 64),
                        kw.pop("dtype", 1))
    p.conv_k = BASE + (1 << 36)
    p.conv_v = BASE + (2 << 36)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _call(p, F=10, S=16, chunk=5, radius=1, rule=0, **ptrs):
    d = dict(q=BASE + (3 << 36), k=BASE + (4 << 36), v=BASE + (5 << 36),
             beta=BASE + (6 << 36), alpha=BASE + (7 << 36), gate=BASE + (8 << 36),
             text=None, out=BASE + (9 << 36))
    d.update(ptrs)
    vp = ctypes.c_void_p
    return hwa.lib().hybrid_attn_fwd(vp(d["q"]), vp(d["k"]), vp(d["v"]), vp(d["beta"]),
                                     vp(d["alpha"]), vp(d["gate"]), vp(d["text"]), F, S,
                                     chunk, radius, rule, vp(d["out"]), None,
                                     ctypes.byref(p))


def _with_ws(p, F=10, S=16, chunk=5, extra=0):
    n = hwa.workspace_bytes(F, S, chunk, p)
    assert n > 0
    p.workspace = BASE + (10 << 36)
    p.workspace_bytes = n + extra
    return p


@no_gpu
def test_argument_validation_codes():
    E = hwa
    p = _with_ws(_params())
    assert _call(p, q=None) == E.HWA_ERR_INVALID_ARG
    assert _call(p, out=None) == E.HWA_ERR_INVALID_ARG
    assert _call(p, beta=None) == E.HWA_ERR_INVALID_ARG
    assert _call(p, F=0) == E.HWA_ERR_INVALID_ARG
    assert _call(p, S=0) == E.HWA_ERR_INVALID_ARG
    assert _call(p, chunk=0) == E.HWA_ERR_INVALID_ARG
    assert _call(p, radius=-1) == E.HWA_ERR_INVALID_ARG
    assert _call(p, rule=3) == E.HWA_ERR_INVALID_ARG
    assert _call(p, q=BASE + 2) == E.HWA_ERR_INVALID_ARG          # misaligned
    assert _call(p, out=BASE + (3 << 36)) == E.HWA_ERR_INVALID_ARG  # out aliases q
    assert _call(p, out=p.workspace) == E.HWA_ERR_INVALID_ARG      # out aliases workspace
    pf = _with_ws(_params(flags=hwa.FLAG_SOFTMAX_ONLY | hwa.FLAG_LINEAR_ONLY))
    assert _call(pf) == E.HWA_ERR_INVALID_ARG
    pf = _with_ws(_params(flags=4))  # no flag asks for the intermediates: bit 4 is unused
    assert _call(pf) == E.HWA_ERR_INVALID_ARG
    pf = _with_ws(_params(flags=64))
    assert _call(pf) == E.HWA_ERR_INVALID_ARG
    assert _call(_with_ws(_params(rms_eps=0.0))) == E.HWA_ERR_INVALID_ARG
    assert _call(_with_ws(_params(c=float("nan")))) == E.HWA_ERR_INVALID_ARG
    # bf16 tiles use 32-bit byte offsets within a head: roundup(N, 64) * d * 2 < 2^31
    pb = _with_ws(_params(head_dim=128, dtype=hwa.HWA_BF16))
    assert _call(pb, F=2048, S=4096) == E.HWA_ERR_INVALID_ARG     # 2^23 tokens
    assert _call(pb, F=2048, S=4095) == E.HWA_ERR_WORKSPACE       # in range, small workspace
    # softmax-only needs no linear-branch inputs but still a workspace
    ps = _params(flags=hwa.FLAG_SOFTMAX_ONLY)
    assert _call(ps, beta=None, alpha=None, gate=None) == E.HWA_ERR_WORKSPACE


@no_gpu
def test_unsupported_and_workspace_codes():
    E = hwa
    assert _call(_params(head_dim=48)) == E.HWA_ERR_UNSUPPORTED
    assert _call(_params(head_dim=16, dtype=1)) == E.HWA_ERR_UNSUPPORTED
    assert _call(_params(dtype=7)) == E.HWA_ERR_INVALID_ARG
    assert _call(_params()) == E.HWA_ERR_WORKSPACE                  # no workspace
    p = _with_ws(_params(), extra=-256)
    assert _call(p) == E.HWA_ERR_WORKSPACE                          # too small
    p = _with_ws(_params())
    p.workspace += 16
    assert _call(p) == E.HWA_ERR_WORKSPACE                          # misaligned
    p = _params()
    p.struct_size = 8
    assert _call(p) == E.HWA_ERR_INVALID_ARG
    assert hwa.lib().hybrid_attn_fwd(None, None, None, None, None, None, None, 10, 16, 5, 1,
                                     0, None, None, None) == E.HWA_ERR_INVALID_ARG


def test_workspace_layout_is_consistent():
    for cfg in inputs.WORKLOADS.values():
        p = hwa.make_params(cfg["batch"], cfg["heads"], cfg["head_dim"],
                            1 if cfg["dtype"] == "bf16" else 0)
        L = hwa.workspace_layout(cfg["frames"], cfg["tokens_per_frame"], cfg["chunk"], p)
        offs = [L[k] for k in ("lohi", "stat_a", "stat_b", "map_m", "bank_p", "bank_q",
                               "decay", "bank_e", "v_t", "st16", "st_eps")]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        assert L["total"] == hwa.workspace_bytes(cfg["frames"], cfg["tokens_per_frame"],
                                                 cfg["chunk"], p)
        B, H, d, F = cfg["batch"], cfg["heads"], cfg["head_dim"], cfg["frames"]
        assert L["stat_b"] - L["stat_a"] >= B * H * F * d * d * 4


@no_gpu
def test_text_state_validation():
    E = hwa
    vp = ctypes.c_void_p
    p = _params()
    L = hwa.lib()
    assert L.hwa_text_state(vp(BASE), vp(BASE + (1 << 36)), vp(BASE + (2 << 36)), 0,
                            vp(BASE + (3 << 36)), None, ctypes.byref(p)) == E.HWA_ERR_INVALID_ARG
    assert L.hwa_text_state(vp(BASE), vp(BASE + (1 << 36)), vp(BASE + (2 << 36)), 16,
                            vp(BASE + (3 << 36)), None, ctypes.byref(p)) == E.HWA_ERR_WORKSPACE
    assert L.hwa_text_state_workspace_bytes(16, ctypes.byref(p)) > 0


@no_gpu
def test_text_state_alignment():
    # the forward's alignment rules: bf16 token rows on 16 bytes, fp32 arrays
    # (beta_txt) on 4; a misaligned slice is rejected before any launch
    E = hwa
    vp = ctypes.c_void_p
    L = hwa.lib()
    p = _params()  # bf16, d 64
    p.workspace = BASE + (10 << 36)
    p.workspace_bytes = L.hwa_text_state_workspace_bytes(16, ctypes.byref(p))
    k, v, b, st = BASE, BASE + (1 << 36), BASE + (2 << 36), BASE + (3 << 36)
    for kk, vv, bb in ((k + 8, v, b), (k, v + 2, b), (k, v, b + 2)):
        assert L.hwa_text_state(vp(kk), vp(vv), vp(bb), 16, vp(st), None,
                                ctypes.byref(p)) == E.HWA_ERR_INVALID_ARG
    pf = _params(dtype=0)  # fp32 rows on 4 bytes
    pf.workspace = BASE + (10 << 36)
    pf.workspace_bytes = L.hwa_text_state_workspace_bytes(16, ctypes.byref(pf))
    assert L.hwa_text_state(vp(k + 2), vp(v), vp(b), 16, vp(st), None,
                            ctypes.byref(pf)) == E.HWA_ERR_INVALID_ARG


@no_gpu
def test_softmax_outputs_validation_and_struct_evolution():
    E = hwa
    # a caller built against the first struct (ending at stage_events) is
    # accepted and its missing fields read as NULL
    p = _params()
    p.struct_size = hwa.Params.softmax_lse.offset
    p.softmax_lse = BASE + (11 << 36)  # beyond the caller's struct: ignored
    assert _call(p) == E.HWA_ERR_WORKSPACE
    p.struct_size = hwa.Params.softmax_lse.offset - 1
    assert _call(p) == E.HWA_ERR_INVALID_ARG
    # outputs of the softmax branch must not overlap out, an input, each other
    p = _with_ws(_params())
    p.softmax_lse = BASE + (9 << 36)                    # = out
    assert _call(p) == E.HWA_ERR_INVALID_ARG
    p.softmax_lse = BASE + (3 << 36)                    # = q
    assert _call(p) == E.HWA_ERR_INVALID_ARG
    p.softmax_lse = BASE + (11 << 36)
    p.softmax_out = BASE + (11 << 36)                   # = softmax_lse
    assert _call(p) == E.HWA_ERR_INVALID_ARG
    p.softmax_out = BASE + (12 << 36) + 2               # misaligned
    assert _call(p) == E.HWA_ERR_INVALID_ARG
    # no softmax branch, nothing to write there
    p = _with_ws(_params(flags=hwa.FLAG_LINEAR_ONLY))
    p.softmax_lse = BASE + (11 << 36)
    assert _call(p) == E.HWA_ERR_INVALID_ARG


def _bwd_call(p, F=10, S=16, chunk=5, radius=1, **ptrs):
    d = dict(q=BASE + (3 << 36), k=BASE + (4 << 36), v=BASE + (5 << 36), o=BASE + (6 << 36),
             lse=BASE + (7 << 36), g=BASE + (8 << 36), dq=BASE + (9 << 36),
             dk=BASE + (11 << 36), dv=BASE + (12 << 36))
    d.update(ptrs)
    vp = ctypes.c_void_p
    return hwa.lib().hwa_softmax_bwd(vp(d["q"]), vp(d["k"]), vp(d["v"]), vp(d["o"]),
                                     vp(d["lse"]), vp(d["g"]), F, S, chunk, radius,
                                     vp(d["dq"]), vp(d["dk"]), vp(d["dv"]), None,
                                     ctypes.byref(p))


def _bwd_ws(p, F=10, S=16, chunk=5, extra=0):
    n = hwa.lib().hwa_softmax_bwd_workspace_bytes(F, S, chunk, ctypes.byref(p))
    assert n > 0
    p.workspace = BASE + (10 << 36)
    p.workspace_bytes = n + extra
    return p


@no_gpu
def test_softmax_bwd_validation():
    E = hwa
    p = _bwd_ws(_params())
    for name in ("q", "k", "v", "o", "lse", "g", "dq", "dk", "dv"):
        assert _bwd_call(p, **{name: None}) == E.HWA_ERR_INVALID_ARG, name
    assert _bwd_call(p, F=0) == E.HWA_ERR_INVALID_ARG
    assert _bwd_call(p, radius=-1) == E.HWA_ERR_INVALID_ARG
    assert _bwd_call(p, q=BASE + 8) == E.HWA_ERR_INVALID_ARG            # misaligned
    assert _bwd_call(p, dk=BASE + (9 << 36)) == E.HWA_ERR_INVALID_ARG   # dk aliases dq
    assert _bwd_call(p, dv=BASE + (5 << 36)) == E.HWA_ERR_INVALID_ARG   # dv aliases v
    assert _bwd_call(p, dq=p.workspace) == E.HWA_ERR_INVALID_ARG        # dq in the workspace
    assert _bwd_call(_bwd_ws(_params(), extra=-256)) == E.HWA_ERR_WORKSPACE
    assert _bwd_call(_params()) == E.HWA_ERR_WORKSPACE
    assert _bwd_call(_params(head_dim=16, dtype=1)) == E.HWA_ERR_UNSUPPORTED


def test_softmax_bwd_workspace_bytes():
    L = hwa.lib()
    for dt in (0, 1):
        p = hwa.make_params(2, 3, 64, dt)
        n = L.hwa_softmax_bwd_workspace_bytes(10, 100, 5, ctypes.byref(p))
        Np = (10 * 100 + 63) // 64 * 64
        # the window table, delta and lse2 per query
        need = 2 * 6 * Np * 4
        assert need <= n <= need + 4 * 256
    assert L.hwa_softmax_bwd_workspace_bytes(0, 100, 5, ctypes.byref(p)) == 0


_LIN = ("q", "k", "v", "beta", "alpha", "gate", "text", "g", "dq", "dk", "dv", "dbeta",
        "dalpha", "dgate", "dtext", "dconv_k", "dconv_v", "drms")


def _lin_call(p, F=10, S=16, chunk=5, radius=1, rule=0, **ptrs):
    d = {n: BASE + ((13 + i) << 36) for i, n in enumerate(_LIN)}
    d.update(ptrs)
    vp = ctypes.c_void_p
    a = [vp(d[n]) for n in _LIN]
    return hwa.lib().hwa_linear_bwd(*a[:8], F, S, chunk, radius, rule, *a[8:], None,
                                    ctypes.byref(p))


def _lin_ws(p, F=10, S=16, chunk=5, extra=0):
    n = hwa.lib().hwa_linear_bwd_workspace_bytes(F, S, chunk, ctypes.byref(p))
    assert n > 0
    p.workspace = BASE + (10 << 36)
    p.workspace_bytes = n + extra
    return p


@no_gpu
def test_linear_bwd_validation():
    E = hwa
    p = _lin_ws(_params())
    for name in _LIN:
        if name in ("text", "dtext", "drms"):  # optional
            continue
        assert _lin_call(p, **{name: None}) == E.HWA_ERR_INVALID_ARG, name
    assert _lin_call(_lin_ws(_params(conv_k=None))) == E.HWA_ERR_INVALID_ARG
    assert _lin_call(p, rule=3) == E.HWA_ERR_INVALID_ARG
    assert _lin_call(p, F=0) == E.HWA_ERR_INVALID_ARG
    assert _lin_call(p, radius=-1) == E.HWA_ERR_INVALID_ARG
    assert _lin_call(p, q=BASE + 8) == E.HWA_ERR_INVALID_ARG              # misaligned bf16
    assert _lin_call(p, dbeta=BASE + 2) == E.HWA_ERR_INVALID_ARG          # misaligned fp32
    assert _lin_call(p, dk=BASE + (21 << 36)) == E.HWA_ERR_INVALID_ARG    # dk aliases dq
    assert _lin_call(p, dbeta=BASE + (16 << 36)) == E.HWA_ERR_INVALID_ARG  # dbeta aliases beta
    assert _lin_call(p, dalpha=p.workspace) == E.HWA_ERR_INVALID_ARG      # in the workspace
    assert _lin_call(p, drms=BASE + (28 << 36)) == E.HWA_ERR_INVALID_ARG  # drms aliases dconv_k
    assert _lin_call(_lin_ws(_params(), extra=-256)) == E.HWA_ERR_WORKSPACE
    assert _lin_call(_params()) == E.HWA_ERR_WORKSPACE
    assert _lin_call(_lin_ws(_params(rms_eps=0.0))) == E.HWA_ERR_INVALID_ARG
    assert _lin_call(_lin_ws(_params(flags=1))) == E.HWA_ERR_INVALID_ARG  # forward-only flag
    assert _lin_call(_params(head_dim=16, dtype=1)) == E.HWA_ERR_UNSUPPORTED


def test_linear_bwd_workspace_bytes():
    L = hwa.lib()
    B, H, d, F, S, chunk = 2, 3, 64, 12, 100, 5
    nch = (F + chunk - 1) // chunk
    bh, dd, N = B * H, d * d * 4, F * S
    for dt in (0, 1):
        p = hwa.make_params(B, H, d, dt)
        n = L.hwa_linear_bwd_workspace_bytes(F, S, chunk, ctypes.byref(p))
        # statistics, inverses, dS_t, the suffix adjoint (F each), both scans'
        # states (F + 1 each), their exponents, the bank gradients, the
        # adjoints of s0, per-frame vectors (gather 2, dalpha, dw), the fp32
        # gradients before the convs, the per-frame tap gradients
        need = (bh * (5 * F + 2 * (F + 1)) * dd + 2 * bh * (F + 1) * d * 4
                + 2 * bh * (nch + 1) * dd + 2 * bh * dd + 4 * bh * F * d * 4
                + 2 * bh * N * d * 4 + bh * F * d * 8 * 4)
        assert need <= n <= need + 16 * 256
    assert L.hwa_linear_bwd_workspace_bytes(0, 100, 5, ctypes.byref(p)) == 0


@no_gpu
def test_noalloc_rejects_before_any_launch():
    # hybrid_attn_fwd_noalloc: sizes whose workspace exceeds the library's
    # fixed scratch array are rejected with HWA_ERR_WORKSPACE, bad arguments
    # with the forward's own codes, all before anything is enqueued
    E = hwa
    vp = ctypes.c_void_p
    fn = hwa.lib().hybrid_attn_fwd_noalloc

    def call(p, F, S, chunk=5, radius=1, **ptrs):
        d = dict(q=BASE + (3 << 36), k=BASE + (4 << 36), v=BASE + (5 << 36),
                 beta=BASE + (6 << 36), alpha=BASE + (7 << 36), gate=BASE + (8 << 36),
                 out=BASE + (9 << 36))
        d.update(ptrs)
        return fn(vp(d["q"]), vp(d["k"]), vp(d["v"]), vp(d["beta"]), vp(d["alpha"]),
                  vp(d["gate"]), None, F, S, chunk, radius, 0, vp(d["out"]), None,
                  ctypes.byref(p))

    cap = 64 << 20
    p = _params(heads=24, head_dim=128)
    assert hwa.workspace_bytes(31, 1560, 5, p) > cap
    assert call(p, 31, 1560) == E.HWA_ERR_WORKSPACE
    assert call(_params(), 0, 16) == E.HWA_ERR_INVALID_ARG
    assert call(_params(head_dim=48), 10, 16) == E.HWA_ERR_UNSUPPORTED
    assert call(_params(), 10, 16, radius=-1) == E.HWA_ERR_INVALID_ARG
    assert call(_params(), 10, 16, q=None) == E.HWA_ERR_INVALID_ARG
    short = _params()
    short.struct_size = hwa.Params.softmax_lse.offset - 1
    assert call(short, 10, 16) == E.HWA_ERR_INVALID_ARG


@no_gpu
def test_frame_alpha_validation():
    E = hwa
    vp = ctypes.c_void_p
    fn = hwa.lib().hwa_frame_alpha
    k, w, b, a, out = (BASE + (i << 36) for i in range(1, 6))

    def call(p, F=10, S=16, **kw):
        d = dict(k=k, w=w, b=b, a=a, out=out)
        d.update(kw)
        return fn(vp(d["k"]), vp(d["w"]), vp(d["b"]), vp(d["a"]), F, S, vp(d["out"]), None,
                  ctypes.byref(p))

    p = _params()
    assert call(p, k=None) == E.HWA_ERR_INVALID_ARG
    assert call(p, out=None) == E.HWA_ERR_INVALID_ARG
    assert call(p, F=0) == E.HWA_ERR_INVALID_ARG
    assert call(p, S=0) == E.HWA_ERR_INVALID_ARG
    assert call(p, k=k + 8) == E.HWA_ERR_INVALID_ARG      # k rows on 16 bytes
    assert call(p, a=a + 2) == E.HWA_ERR_INVALID_ARG      # fp32 on 4 bytes
    assert call(p, out=w) == E.HWA_ERR_INVALID_ARG        # alpha overlaps W
    assert call(p, out=k + 64) == E.HWA_ERR_INVALID_ARG   # alpha inside k
    assert call(_params(head_dim=48)) == E.HWA_ERR_UNSUPPORTED


@no_gpu
def test_routed_flag_validation():
    E = hwa
    R = hwa.FLAG_ROUTED
    p = _with_ws(_params(flags=R))
    p.route_tau = float("nan")
    assert _call(p) == E.HWA_ERR_INVALID_ARG                       # NaN threshold
    p = _with_ws(_params(flags=R | hwa.FLAG_LINEAR_ONLY))
    assert _call(p) == E.HWA_ERR_INVALID_ARG                       # no softmax branch
    p = _with_ws(_params(flags=R, dtype=0))
    assert _call(p) == E.HWA_ERR_UNSUPPORTED                       # fp32
    p = _params(flags=R)
    p.struct_size = hwa.Params.route_tau.offset                    # struct ends before tau
    assert _call(p) == E.HWA_ERR_INVALID_ARG
    p = _with_ws(_params(flags=R, head_dim=128), F=40, S=30000)
    assert _call(p, F=40, S=30000) == E.HWA_ERR_UNSUPPORTED        # window > 4096 tiles
    # the routed layout needs more workspace than the dense one
    pd, pr = _params(), _params(flags=R)
    assert hwa.workspace_bytes(10, 16, 5, pr) > hwa.workspace_bytes(10, 16, 5, pd)
    L = hwa.route_layout(10, 16, 5, pr)
    assert L["tiles_per_chunk"] == 1 and L["stride"] == 160 // 128 + 2
