"""Pins for the oracle's dropout of the attention weights.

The SDPA node call in the cuDNN 9 blog ("SDPA usage") has a ``dropout``
option without semantics. Reading: P_ij is multiplied by Z_ij, with Z from a
counter-based Philox4x32-10 stream keyed by the seed (``dropout_mask``). Pins:
the Philox known-answer vectors published with the Random123 library, keep
statistics, p = 0 and p = 1 limits, independence from row blocking, a scalar
re-derivation of each mask byte, torch float64 autograd on the same fixed mask,
and finite differences (with the mask fixed the loss is smooth).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_forward, dropout_keep_threshold, dropout_mask, philox4x32_10


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("ctr,key,expect", [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
])
def test_philox_known_answers(ctr, key, expect):
    out = philox4x32_10(*[np.array([c], dtype=np.uint64) for c in ctr], np.array([key[0]]), np.array([key[1]]))
    assert tuple(int(o[0]) for o in out) == expect


def test_mask_bytes_by_scalar_rule():
    """Each element's byte re-derived one at a time from the stated rule."""
    bh, seed, offset, p = 5, 0x1234_5678_9ABC_DEF0, 11, 0.3
    z = dropout_mask(bh, np.arange(9), 13, p, seed, offset)
    k8 = dropout_keep_threshold(p)
    for i in range(9):
        for j in range(13):
            w = philox4x32_10(np.array([j // 4]), np.array([i // 4]), np.array([bh]), np.array([offset]),
                              np.array([seed & 0xFFFFFFFF]), np.array([seed >> 32]))
            byte = (int(w[i % 4][0]) >> (8 * (j % 4))) & 0xFF
            assert z[i, j] == (256.0 / k8 if byte < k8 else 0.0)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_statistics(p):
    z = dropout_mask(3, np.arange(512), 2048, p, 99, 1)
    k8 = dropout_keep_threshold(p)
    keep = (z > 0).mean()
    sigma = math.sqrt(k8 / 256 * (1 - k8 / 256) / z.size)
    assert abs(keep - k8 / 256) < 6 * sigma
    assert abs(z.mean() - 1.0) < 6 * sigma * 256 / max(k8, 1)
    assert abs(k8 / 256 - (1 - p)) <= 1 / 512


def test_limits_and_blocking():
    rng = np.random.default_rng(51)
    q, k, v = (_rand(rng, 2, 2, 33, 8) for _ in range(3))
    o0, l0 = attention_forward(q, k, v, 0.3, True)
    o1, l1 = attention_forward(q, k, v, 0.3, True, dropout_p=0.0, dropout_seed=5)
    np.testing.assert_array_equal(o0, o1)
    o2, l2 = attention_forward(q, k, v, 0.3, True, dropout_p=1.0, dropout_seed=5)
    assert (o2 == 0).all()
    np.testing.assert_allclose(l2, l0, atol=1e-12)  # LSE is that of the undropped weights
    oa, _ = attention_forward(q, k, v, 0.3, True, row_block=5, dropout_p=0.4, dropout_seed=7, dropout_offset=3)
    ob, _ = attention_forward(q, k, v, 0.3, True, row_block=64, dropout_p=0.4, dropout_seed=7, dropout_offset=3)
    np.testing.assert_allclose(oa, ob, atol=1e-12)
    oc, _ = attention_forward(q, k, v, 0.3, True, dropout_p=0.4, dropout_seed=7, dropout_offset=4)
    assert not np.allclose(oa, oc)  # a new offset draws a new mask


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_against_torch_autograd(causal):
    """O = (softmax(S) * Z) V and its gradients via torch float64 autograd, with
    the oracle's own mask Z as a constant."""
    rng = np.random.default_rng(52 + causal)
    b, h_q, h_kv, s, d = 2, 4, 2, 11, 5
    q, k, v = _rand(rng, b, h_q, s, d), _rand(rng, b, h_kv, s, d), _rand(rng, b, h_kv, s, d)
    do = _rand(rng, b, h_q, s, d)
    kw = dict(dropout_p=0.35, dropout_seed=2024, dropout_offset=9)
    z = np.stack([np.stack([dropout_mask(bi * h_q + hq, np.arange(s), s, 0.35, 2024, 9) for hq in range(h_q)])
                  for bi in range(b)])
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(h_q // h_kv, dim=1)
    vv = tv.repeat_interleave(h_q // h_kv, dim=1)
    sc = 0.4 * tq @ kk.transpose(-1, -2)
    if causal:
        sc = sc.masked_fill(torch.triu(torch.ones(s, s, dtype=torch.bool), 1), float("-inf"))
    to = (torch.softmax(sc, dim=-1) * torch.tensor(z)) @ vv
    (to * torch.tensor(do)).sum().backward()
    o, _ = attention_forward(q, k, v, 0.4, causal, **kw)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    dq, dk, dv = attention_backward(q, k, v, do, 0.4, causal, **kw)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_dropout_backward_matches_finite_differences():
    rng = np.random.default_rng(53)
    q, k, v = _rand(rng, 1, 2, 6, 3), _rand(rng, 1, 2, 7, 3), _rand(rng, 1, 2, 7, 3)
    do = _rand(rng, 1, 2, 6, 3)
    kw = dict(dropout_p=0.5, dropout_seed=77, dropout_offset=0, align="bottom_right")

    def loss(q_, k_, v_):
        return float((attention_forward(q_, k_, v_, 0.6, True, **kw)[0] * do).sum())

    dq, dk, dv = attention_backward(q, k, v, do, 0.6, True, **kw)
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
