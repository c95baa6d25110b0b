"""Whole-call pins of the oracle (CPU only).

"Why video models are stuck on attention" (VDN-H3 article): the softmax branch
covers the window, the linear branch everything outside it, and the outputs
are summed.
"""

import numpy as np
import pytest

import oracle
from hybrid_window_softmax_amd import inputs


def _run(inp, rule="vdn_solve", text=True, flip=False):
    cfg = inp.cfg
    B, H = cfg["batch"], cfg["heads"]
    F, S, d = cfg["frames"], cfg["tokens_per_frame"], cfg["head_dim"]
    outs = []
    for b in range(B):
        for h in range(H):
            args = [inp.f64(n, b, h) for n in ("q", "k", "v")]
            beta, alpha, gate = inp.beta[b, h].astype(np.float64), inp.alpha[b, h].astype(np.float64), inp.f64("gate", b, h)
            st = None
            if text and inp.k_txt is not None:
                st = oracle.text_state(inp.f64("k_txt", b, h), inp.f64("v_txt", b, h), inp.beta_txt[b, h])
            if flip:  # reverse the frame order, keep token order within frames
                def fl(x, per_token=True):
                    if per_token:
                        return x.reshape(F, S, *x.shape[1:])[::-1].reshape(x.shape)
                    return x[::-1]
                args = [fl(a) for a in args]
                beta, gate, alpha = fl(beta), fl(gate), fl(alpha, False)
            r = oracle.hybrid_attn_head(*args, beta, alpha, gate, st, inp.conv_k[h], inp.conv_v[h],
                                        inp.rms_weight, S, cfg["chunk"], cfg["radius"], rule,
                                        cfg["c"], 0.5, 1e-6)
            outs.append(r)
    return outs


def test_tiny_workload_has_no_far_field():
    inp = inputs.make("tiny-f32")
    (out, o_sm, y, _), = _run(inp)
    # F = 10 frames with chunk 5, radius 1: every window is [0, 9] and there is
    # no text state, so the linear branch reads a zero state: y == 0 exactly
    assert not np.any(y)
    assert np.array_equal(out, o_sm)


def test_beta0_no_text_is_pure_softmax():
    cfg = inputs.tiny_config(frames=17, text_tokens=0)
    inp = inputs.make(cfg, beta_zero=True)
    (out, o_sm, y, _), = _run(inp)
    assert not np.any(y)
    assert np.array_equal(out, o_sm)


@pytest.mark.parametrize("rule", oracle.RULES)
def test_whole_frame_reversal_symmetry(rule):
    # with F a multiple of chunk the window geometry is mirror-symmetric, so
    # reversing the frames reverses the output (prefix and suffix swap roles)
    cfg = inputs.tiny_config(frames=15, text_tokens=8, rule=rule)
    inp = inputs.make(cfg)
    (out, o_sm, y, _), = _run(inp, rule)
    (outr, o_smr, yr, _), = _run(inp, rule, flip=True)
    F, S = cfg["frames"], cfg["tokens_per_frame"]
    back = lambda x: x.reshape(F, S, -1)[::-1].reshape(x.shape)  # noqa: E731
    assert np.abs(back(o_smr) - o_sm).max() < 1e-12
    assert np.abs(back(yr) - y).max() < 1e-9
    assert np.any(y)


def test_rel_frobenius_semantics():
    a = np.ones((3, 4))
    assert oracle.rel_frobenius(a, a) == 0.0
    assert abs(oracle.rel_frobenius(1.5 * a, a) - 0.5) < 1e-15
    assert oracle.rel_frobenius(np.zeros(3), np.zeros(3)) == 0.0
    assert oracle.rel_frobenius(np.array([1e-30, 0, 0]), np.zeros(3)) == float("inf")


@pytest.mark.parametrize("workers", [1, 3])
def test_whole_call_wrapper_is_the_slice_definition(workers):
    # the [B, H] wrapper (task split over (b, h, query chunk) and (b, h), run
    # in one process or a pool) equals the one-slice definition for every
    # (b, h): per-head conv taps, per-slice text states and alpha, a partial
    # last chunk, and separate softmax-branch q/k for the softmax tasks
    cfg = inputs.tiny_config(frames=12, text_tokens=8, head_dim=16, tokens_per_frame=10,
                             heads=2, batch=2, chunk=5, seed=301)
    inp = inputs.make(cfg, random_rms_weight=True)
    other = inputs.make({**cfg, "seed": 302})
    B, H, F, S = cfg["batch"], cfg["heads"], cfg["frames"], cfg["tokens_per_frame"]
    f64 = lambda name, src=inp: src.f32(name).astype(np.float64)  # noqa: E731
    st = np.stack([np.stack([oracle.text_state(inp.f64("k_txt", b, h), inp.f64("v_txt", b, h),
                                               inp.beta_txt[b, h]) for h in range(H)])
                   for b in range(B)])
    assert not np.allclose(inp.conv_k[0], inp.conv_k[1])
    assert not np.allclose(st[0, 0], st[1, 1]) and not np.allclose(inp.alpha[0, 1], inp.alpha[1, 1])
    for rope in (False, True):
        qr = f64("q", other) if rope else None
        kr = f64("k", other) if rope else None
        out, o_sm, y = oracle.hybrid_attn(
            f64("q"), f64("k"), f64("v"), inp.beta.astype(np.float64),
            inp.alpha.astype(np.float64), f64("gate"), st, inp.conv_k, inp.conv_v,
            inp.rms_weight, F, S, cfg["chunk"], cfg["radius"], "vdn_scaled", 0.5, 0.5, 1e-6,
            q_rope=qr, k_rope=kr, workers=workers)
        for b in range(B):
            for h in range(H):
                ref = oracle.hybrid_attn_head(
                    inp.f64("q", b, h), inp.f64("k", b, h), inp.f64("v", b, h),
                    inp.beta[b, h], inp.alpha[b, h], inp.f64("gate", b, h), st[b, h],
                    inp.conv_k[h], inp.conv_v[h], inp.rms_weight, S, cfg["chunk"],
                    cfg["radius"], "vdn_scaled", 0.5, 0.5, 1e-6,
                    q_rope=None if qr is None else qr[b, h],
                    k_rope=None if kr is None else kr[b, h])
                for got, r in ((out, ref[0]), (o_sm, ref[1]), (y, ref[2])):
                    assert np.allclose(got[b, h], r, rtol=1e-12, atol=1e-15), (rope, b, h)
        assert np.any(y) and np.array_equal(out, o_sm + y)
    # without a text state and with the default (unit) RMSNorm weight
    out, o_sm, y = oracle.hybrid_attn(
        f64("q"), f64("k"), f64("v"), inp.beta.astype(np.float64),
        inp.alpha.astype(np.float64), f64("gate"), None, inp.conv_k, inp.conv_v, None, F, S,
        workers=workers)
    ref = oracle.hybrid_attn_head(inp.f64("q", 1, 0), inp.f64("k", 1, 0), inp.f64("v", 1, 0),
                                  inp.beta[1, 0], inp.alpha[1, 0], inp.f64("gate", 1, 0), None,
                                  inp.conv_k[0], inp.conv_v[0], np.ones(16), S)
    assert np.allclose(out[1, 0], ref[0], rtol=1e-12, atol=1e-15)
