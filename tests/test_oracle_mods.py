"""Pins for the oracle's score modifiers: an additive bias tensor and ALiBi.

The cuDNN 9 blog's SDPA node call ("SDPA usage") lists ``bias`` and
``use_alibi_mask`` options without semantics. The oracle's reading: both are
added to the scaled scores before the mask and the softmax; ALiBi adds
-slope[h] * |i + off - j| with the ALiBi paper's slopes. Pinned against
scalar brute force, torch's float64 SDPA with a float attn_mask (which torch
adds to the scaled scores), softmax invariances, mask equivalence, the ALiBi
paper's closed-form slopes, and finite differences.
"""
import math

import numpy as np
import pytest
import torch

from oracle import alibi_slopes, attention_backward, attention_forward


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def brute_mod(q, k, v, scale, causal, bias, slopes):
    b, h_q, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    grp = h_q // h_kv
    out = np.zeros((b, h_q, s_q, d))
    lse = np.zeros((b, h_q, s_q))
    for bi in range(b):
        for hq in range(h_q):
            g = hq // grp
            for i in range(s_q):
                keys = [j for j in range(s_kv) if not causal or j <= i]
                sc = []
                for j in keys:
                    x = scale * math.fsum(float(q[bi, hq, i, t]) * float(k[bi, g, j, t]) for t in range(d))
                    if bias is not None:
                        x += float(bias[bi % bias.shape[0], hq % bias.shape[1], i, j])
                    if slopes is not None:
                        x -= float(slopes[hq]) * abs(i - j)
                    sc.append(x)
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                l = math.fsum(e)
                for t in range(d):
                    out[bi, hq, i, t] = math.fsum(e[n] * float(v[bi, g, j, t]) for n, j in enumerate(keys)) / l
                lse[bi, hq, i] = m + math.log(l)
    return out, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bias_shape", [None, (2, 4), (1, 4), (2, 1), (1, 1)])
@pytest.mark.parametrize("use_alibi", [False, True])
def test_modifiers_match_brute_force(causal, bias_shape, use_alibi):
    rng = np.random.default_rng(31 + causal + 2 * use_alibi)
    b, h_q, h_kv, s_q, s_kv, d = 2, 4, 2, 6, 6, 3
    q, k, v = _rand(rng, b, h_q, s_q, d), _rand(rng, b, h_kv, s_kv, d), _rand(rng, b, h_kv, s_kv, d)
    bias = None if bias_shape is None else _rand(rng, *bias_shape, s_q, s_kv)
    slopes = alibi_slopes(h_q) if use_alibi else None
    o, l = attention_forward(q, k, v, 0.5, causal, row_block=4, bias=bias, alibi_slopes=slopes)
    ob, lb = brute_mod(q, k, v, 0.5, causal, bias, slopes)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


def test_alibi_slopes_closed_form():
    """The ALiBi paper: 8 heads get 1/2, 1/4, ..., 1/256; 16 heads interleave
    the 8-head slopes with their geometric means; 12 heads take the 8-head
    slopes and then every other slope of 16 heads."""
    np.testing.assert_allclose(alibi_slopes(8), [2.0 ** -(i + 1) for i in range(8)], rtol=1e-15)
    s16 = alibi_slopes(16)
    np.testing.assert_allclose(s16[1::2], alibi_slopes(8), rtol=1e-15)
    np.testing.assert_allclose(s16[0::2], [2.0 ** -(i + 0.5) for i in range(8)], rtol=1e-15)
    np.testing.assert_allclose(alibi_slopes(12), list(alibi_slopes(8)) + list(s16[0::2][:4]), rtol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_modifiers_against_torch_float_mask(causal):
    """torch's SDPA adds a float attn_mask to the scaled scores: bias + ALiBi
    built explicitly, float64, forward and backward (bias without gradient)."""
    rng = np.random.default_rng(41 + causal)
    b, h, s, d = 2, 4, 13, 8
    q, k, v, do = (_rand(rng, b, h, s, d) for _ in range(4))
    bias = _rand(rng, 1, h, s, s)
    slopes = alibi_slopes(h)
    i = np.arange(s)
    alibi = -slopes[:, None, None] * np.abs(i[:, None] - i[None, :])[None]
    full = bias + alibi[None]
    if causal:
        full = np.where(i[None, None, None, :] <= i[None, None, :, None], full, -np.inf)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(full), scale=0.3)
    (to * torch.tensor(do)).sum().backward()
    o, _ = attention_forward(q, k, v, 0.3, causal, bias=bias, alibi_slopes=slopes)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    dq, dk, dv = attention_backward(q, k, v, do, 0.3, causal, bias=bias, alibi_slopes=slopes)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_row_constant_bias_shifts_lse_only():
    rng = np.random.default_rng(43)
    q, k, v = _rand(rng, 1, 2, 7, 4), _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4)
    c = _rand(rng, 1, 2, 7, 1) * 3
    bias = np.broadcast_to(c, (1, 2, 7, 9))
    o0, l0 = attention_forward(q, k, v, 0.5, False)
    o1, l1 = attention_forward(q, k, v, 0.5, False, bias=bias)
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(l1, l0 + c[..., 0], atol=1e-12)


def test_minus_infinity_bias_equals_causal_mask():
    rng = np.random.default_rng(44)
    q, k, v = (_rand(rng, 2, 3, 8, 5) for _ in range(3))
    i = np.arange(8)
    bias = np.where(i[None, :] <= i[:, None], 0.0, -np.inf)[None, None]
    o0, l0 = attention_forward(q, k, v, 0.4, True)
    o1, l1 = attention_forward(q, k, v, 0.4, False, bias=bias)
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(l1, l0, atol=1e-12)


@pytest.mark.parametrize("align", ["top_left", "bottom_right"])
def test_alibi_equals_explicit_bias(align):
    rng = np.random.default_rng(45)
    b, h, s_q, s_kv, d = 1, 4, 5, 11, 4
    q, k, v = _rand(rng, b, h, s_q, d), _rand(rng, b, h, s_kv, d), _rand(rng, b, h, s_kv, d)
    slopes = alibi_slopes(h)
    off = (s_kv - s_q) if align == "bottom_right" else 0
    dist = np.abs(np.arange(s_q)[:, None] + off - np.arange(s_kv)[None, :])
    bias = (-slopes[:, None, None] * dist[None])[None]
    o0, l0 = attention_forward(q, k, v, 0.6, True, align=align, alibi_slopes=slopes)
    o1, l1 = attention_forward(q, k, v, 0.6, True, align=align, bias=bias)
    np.testing.assert_allclose(o0, o1, atol=1e-12)
    np.testing.assert_allclose(l0, l1, atol=1e-12)


def test_modified_backward_matches_finite_differences():
    rng = np.random.default_rng(46)
    b, h_q, h_kv, s_q, s_kv, d = 1, 2, 1, 5, 6, 3
    q, k, v = _rand(rng, b, h_q, s_q, d), _rand(rng, b, h_kv, s_kv, d), _rand(rng, b, h_kv, s_kv, d)
    do = _rand(rng, b, h_q, s_q, d)
    kw = dict(bias=_rand(rng, 1, h_q, s_q, s_kv), alibi_slopes=alibi_slopes(h_q), align="bottom_right")

    def loss(q_, k_, v_):
        return float((attention_forward(q_, k_, v_, 0.7, True, **kw)[0] * do).sum())

    dq, dk, dv = attention_backward(q, k, v, do, 0.7, True, **kw)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            plus = {"q": q, "k": k, "v": v, name: xp}
            minus = {"q": q, "k": k, "v": v, name: xm}
            num[idx] = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / (2 * eps)
        err = np.abs(num - g).max() / max(1e-12, np.abs(g).max())
        assert err < 1e-6, (name, err)
