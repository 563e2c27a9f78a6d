"""Pins for the oracle's padding mask (per-batch seq_len_q / seq_len_kv) and
bottom-right causal alignment.

The cuDNN 9 blog's SDPA node call ("SDPA usage") lists ``use_padding_mask``
with per-batch ``seq_len_q`` / ``seq_len_kv`` next to ``use_causal_mask``; the
pages give no further semantics. The oracle's readings: batch element b uses
its first seq_len_q[b] rows and seq_len_kv[b] keys; bottom-right causal lets
row i see keys j <= i + (lk - lq); a row that sees no key has O = 0,
LSE = -inf and no gradient. These tests pin the implementation of those
readings against brute force, against the unpadded problem, against torch's
own lower-right causal bias and against finite differences.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_forward, attention_probs


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _lse_close(a, b, atol=1e-12):
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    fin = np.isfinite(b)
    np.testing.assert_allclose(a[fin], b[fin], rtol=0, atol=atol)


def brute_masked(q, k, v, scale, causal, lens_q, lens_kv, bottom_right):
    """Scalar loops with math.exp / math.fsum; the visibility rule is written out here."""
    b, h_q, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    grp = h_q // h_kv
    out = np.zeros((b, h_q, s_q, d))
    lse = np.full((b, h_q, s_q), -np.inf)
    for bi in range(b):
        lq, lk = lens_q[bi], lens_kv[bi]
        shift = (lk - lq) if (causal and bottom_right) else 0
        for hq in range(h_q):
            g = hq // grp
            for i in range(lq):
                keys = [j for j in range(lk) if not causal or j - shift <= i]
                if not keys:
                    continue
                sc = [scale * math.fsum(float(q[bi, hq, i, t]) * float(k[bi, g, j, t]) for t in range(d))
                      for j in keys]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                l = math.fsum(e)
                for t in range(d):
                    out[bi, hq, i, t] = math.fsum(e[n] * float(v[bi, g, j, t]) for n, j in enumerate(keys)) / l
                lse[bi, hq, i] = m + math.log(l)
    return out, lse


@pytest.mark.parametrize("causal,bottom_right", [(False, False), (True, False), (True, True)])
@pytest.mark.parametrize("dims", [(2, 2, 1, 7, 9, 3), (3, 2, 2, 9, 5, 4)])
def test_padded_forward_matches_brute_force(dims, causal, bottom_right):
    b, h_q, h_kv, s_q, s_kv, d = dims
    rng = np.random.default_rng(sum(dims) + 2 * causal + bottom_right)
    q, k, v = _rand(rng, b, h_q, s_q, d), _rand(rng, b, h_kv, s_kv, d), _rand(rng, b, h_kv, s_kv, d)
    lens_q = [s_q, 0, 3][:b] if b == 3 else [s_q - 2, 4]
    lens_kv = [s_kv - 1, 2, s_kv][:b] if b == 3 else [s_kv, 1]
    align = "bottom_right" if bottom_right else "top_left"
    o, l = attention_forward(q, k, v, 0.45, causal, row_block=4, seq_len_q=np.array(lens_q),
                             seq_len_kv=np.array(lens_kv), align=align)
    ob, lb = brute_masked(q, k, v, 0.45, causal, lens_q, lens_kv, bottom_right)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    _lse_close(l, lb)


@pytest.mark.parametrize("bottom_right", [False, True])
def test_padded_equals_unpadded_slice(bottom_right):
    """Each batch element equals the oracle run on its unpadded slice alone."""
    rng = np.random.default_rng(21 + bottom_right)
    b, h_q, h_kv, s_q, s_kv, d = 3, 4, 2, 12, 15, 5
    q, k, v = _rand(rng, b, h_q, s_q, d), _rand(rng, b, h_kv, s_kv, d), _rand(rng, b, h_kv, s_kv, d)
    do = _rand(rng, b, h_q, s_q, d)
    lq, lk = np.array([12, 5, 9]), np.array([15, 11, 4])
    align = "bottom_right" if bottom_right else "top_left"
    o, l = attention_forward(q, k, v, 0.3, True, seq_len_q=lq, seq_len_kv=lk, align=align)
    dq, dk, dv = attention_backward(q, k, v, do, 0.3, True, seq_len_q=lq, seq_len_kv=lk, align=align)
    for bi in range(b):
        a, c = lq[bi], lk[bi]
        sl = lambda x, n: x[bi:bi + 1, :, :n]
        o1, l1 = attention_forward(sl(q, a), sl(k, c), sl(v, c), 0.3, True, align=align)
        dq1, dk1, dv1 = attention_backward(sl(q, a), sl(k, c), sl(v, c), sl(do, a), 0.3, True, align=align)
        np.testing.assert_allclose(o[bi, :, :a], o1[0], atol=1e-12)
        _lse_close(l[bi, :, :a], l1[0])
        np.testing.assert_allclose(dq[bi, :, :a], dq1[0], atol=1e-12)
        np.testing.assert_allclose(dk[bi, :, :c], dk1[0], atol=1e-12)
        np.testing.assert_allclose(dv[bi, :, :c], dv1[0], atol=1e-12)
        # padded rows and keys: zero output, -inf LSE, zero gradients
        assert (o[bi, :, a:] == 0).all() and np.isneginf(l[bi, :, a:]).all()
        assert (dq[bi, :, a:] == 0).all() and (dk[bi, :, c:] == 0).all() and (dv[bi, :, c:] == 0).all()


def test_padding_ignores_values_beyond_lengths():
    rng = np.random.default_rng(23)
    b, h, s_q, s_kv, d = 2, 2, 10, 13, 4
    q, k, v = _rand(rng, b, h, s_q, d), _rand(rng, b, h, s_kv, d), _rand(rng, b, h, s_kv, d)
    lq, lk = np.array([6, 10]), np.array([13, 7])
    o, l = attention_forward(q, k, v, 0.5, True, seq_len_q=lq, seq_len_kv=lk, align="bottom_right")
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[0, :, 6:] = 1e3
    k2[1, :, 7:] = -50.0
    v2[1, :, 7:] = np.nan
    o2, l2 = attention_forward(q2, k2, v2, 0.5, True, seq_len_q=lq, seq_len_kv=lk, align="bottom_right")
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_bottom_right_equals_top_left_when_square():
    rng = np.random.default_rng(24)
    q, k, v = _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4)
    o1, l1 = attention_forward(q, k, v, 0.6, True, align="top_left")
    o2, l2 = attention_forward(q, k, v, 0.6, True, align="bottom_right")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("s_q,s_kv", [(4, 11), (11, 4), (7, 7)])
def test_bottom_right_against_torch_lower_right_bias(s_q, s_kv):
    """torch's causal_lower_right bias (its own definition of the bottom-right
    diagonal), float64 CPU SDPA, forward and backward; torch returns NaN rows
    for rows that see no key, where the oracle's reading gives 0."""
    from torch.nn.attention.bias import causal_lower_right

    rng = np.random.default_rng(25 + s_q)
    b, h, d = 2, 3, 6
    q, k, v = _rand(rng, b, h, s_q, d), _rand(rng, b, h, s_kv, d), _rand(rng, b, h, s_kv, d)
    do = _rand(rng, b, h, s_q, d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = causal_lower_right(s_q, s_kv)._materialize(torch.device("cpu"))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.4)
    rows = mask.any(dim=-1).numpy()  # rows that see at least one key
    (torch.nan_to_num(to) * torch.tensor(do)).sum().backward()
    o, _ = attention_forward(q, k, v, 0.4, True, align="bottom_right")
    np.testing.assert_allclose(o[:, :, rows], to.detach().numpy()[:, :, rows], atol=1e-12)
    assert (o[:, :, ~rows] == 0).all()
    if rows.all():  # torch's gradient through NaN rows is NaN; compare only fully defined cases
        dq, dk, dv = attention_backward(q, k, v, do, 0.4, True, align="bottom_right")
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_padding_against_torch_boolean_mask():
    """torch float64 SDPA with an explicit boolean mask built from the lengths
    (rows of valid queries only)."""
    rng = np.random.default_rng(26)
    b, h, s_q, s_kv, d = 3, 2, 8, 10, 5
    q, k, v = _rand(rng, b, h, s_q, d), _rand(rng, b, h, s_kv, d), _rand(rng, b, h, s_kv, d)
    lq, lk = np.array([8, 3, 6]), np.array([10, 10, 2])
    o, _ = attention_forward(q, k, v, 0.5, False, seq_len_q=lq, seq_len_kv=lk)
    for bi in range(b):
        mask = torch.zeros(s_q, s_kv, dtype=torch.bool)
        mask[:, :lk[bi]] = True
        to = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[bi]), torch.tensor(k[bi]), torch.tensor(v[bi]), attn_mask=mask, scale=0.5)
        np.testing.assert_allclose(o[bi, :, :lq[bi]], to.numpy()[:, :lq[bi]], atol=1e-12)


def test_probs_rows_sum_to_one_or_zero():
    rng = np.random.default_rng(27)
    q, k = _rand(rng, 2, 2, 9, 3), _rand(rng, 2, 2, 5, 3)
    p = attention_probs(q, k, 0.7, True, seq_len_q=np.array([9, 4]), seq_len_kv=np.array([5, 3]),
                        align="bottom_right")
    sums = p.sum(axis=-1)
    # bottom-right, batch 0: lq 9, lk 5 -> rows 0..3 see nothing; batch 1: lq 4, lk 3 -> row 0 sees nothing
    expect = np.ones((2, 2, 9))
    expect[0, :, :4] = 0
    expect[1, :, 0] = 0
    expect[1, :, 4:] = 0
    np.testing.assert_allclose(sums, expect, atol=1e-12)


def test_padded_backward_matches_finite_differences():
    """Central differences of L = sum(O * dO) with padding and bottom-right
    rows that see no key (their O is constant 0, so they carry no gradient)."""
    rng = np.random.default_rng(28)
    b, h_q, h_kv, s_q, s_kv, d = 2, 2, 1, 6, 4, 3
    q, k, v = _rand(rng, b, h_q, s_q, d), _rand(rng, b, h_kv, s_kv, d), _rand(rng, b, h_kv, s_kv, d)
    do = _rand(rng, b, h_q, s_q, d)
    kw = dict(seq_len_q=np.array([6, 4]), seq_len_kv=np.array([4, 3]), align="bottom_right")

    def loss(q_, k_, v_):
        return float((attention_forward(q_, k_, v_, 0.9, True, **kw)[0] * do).sum())

    dq, dk, dv = attention_backward(q, k, v, do, 0.9, True, **kw)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            plus = {"q": q, "k": k, "v": v, name: xp}
            minus = {"q": q, "k": k, "v": v, name: xm}
            num[idx] = (loss(plus["q"], plus["k"], plus["v"])
                        - loss(minus["q"], minus["k"], minus["v"])) / (2 * eps)
        err = np.abs(num - g).max() / max(1e-12, np.abs(g).max())
        assert err < 1e-6, (name, err)
    assert (dq[0, :, :2] == 0).all()  # rows 0, 1 of batch 0 see no key (lq 6, lk 4)
