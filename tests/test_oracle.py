"""Pins for the float64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a scalar
brute force, closed forms, invariants the definition fixes, finite
differences, a library routine (torch's SDPA in float64 on the CPU), and the
shapes / layouts the pages print (tests/golden/pages_printed_values.json).
A plausible slip in the oracle (a dropped scale, a flipped mask, log2 for ln,
interleaved head groups, a missing D term or scale in the backward, a wrong
fp8 exponent bias) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import sdpa_inputs
from oracle import (attention_backward, attention_forward, attention_probs,
                    fp8_dequantize, fp8_e4m3_decode, fp8_e5m2_decode)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# Brute force: scalar loops with math.exp / math.fsum (JAX attention codelab,
# step 1: scores, scale + softmax, weights times V).
# --------------------------------------------------------------------------
def brute_forward(q, k, v, scale, causal):
    b, h_q, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    grp = h_q // h_kv
    out = np.zeros((b, h_q, s_q, d))
    lse = np.zeros((b, h_q, s_q))
    for bi in range(b):
        for hq in range(h_q):
            g = hq // grp
            for i in range(s_q):
                keys = [j for j in range(s_kv) if (not causal or j <= i)]
                sc = [scale * math.fsum(float(q[bi, hq, i, t]) * float(k[bi, g, j, t]) for t in range(d))
                      for j in keys]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                l = math.fsum(e)
                for t in range(d):
                    out[bi, hq, i, t] = math.fsum(e[n] * float(v[bi, g, j, t]) for n, j in enumerate(keys)) / l
                lse[bi, hq, i] = m + math.log(l)
    return out, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 5, 5, 3), (2, 4, 2, 7, 7, 4), (1, 3, 1, 6, 9, 8),
                                   (1, 2, 2, 9, 4, 2)])
def test_forward_matches_brute_force(shape, causal):
    b, h_q, h_kv, s_q, s_kv, d = shape
    rng = np.random.default_rng(sum(shape) + causal)
    q, k, v = _rand(rng, b, h_q, s_q, d), _rand(rng, b, h_kv, s_kv, d), _rand(rng, b, h_kv, s_kv, d)
    scale = 0.37
    o, l = attention_forward(q, k, v, scale, causal, row_block=3)
    ob, lb = brute_forward(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


def test_closed_form_two_keys():
    """One query, two keys, d=1: P = (e^{s a x}, e^{s a y}) / sum, computed by hand."""
    a, x, y, u, w, s = 1.5, 0.8, -0.4, 2.0, -1.0, 0.9
    q = np.array([[[[a]]]])
    k = np.array([[[[x], [y]]]])
    v = np.array([[[[u], [w]]]])
    o, l = attention_forward(q, k, v, s, False)
    p0 = 1.0 / (1.0 + math.exp(s * a * (y - x)))
    assert abs(o[0, 0, 0, 0] - (p0 * u + (1 - p0) * w)) < 1e-14
    assert abs(l[0, 0, 0] - math.log(math.exp(s * a * x) + math.exp(s * a * y))) < 1e-14


# --------------------------------------------------------------------------
# Invariants fixed by the definition.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    rng = np.random.default_rng(1)
    q, k = _rand(rng, 2, 4, 11, 8), _rand(rng, 2, 2, 11, 8)
    p = attention_probs(q, k, 0.3, causal)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)
    assert (p >= 0).all()
    if causal:
        assert np.all(np.triu(p[0, 0], 1) == 0.0)


def test_causal_first_row_is_v0():
    """Causal row 0 sees only key 0: O_0 = V_0, LSE_0 = scale q0.k0, dQ_0 = 0."""
    rng = np.random.default_rng(2)
    q, k, v, do = (_rand(rng, 1, 2, 8, 5) for _ in range(4))
    scale = 0.21
    o, l = attention_forward(q, k, v, scale, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(l[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               atol=1e-14)
    dq, _, _ = attention_backward(q, k, v, do, scale, True)
    np.testing.assert_allclose(dq[:, :, 0], 0.0, atol=1e-15)


def test_causal_last_row_equals_full():
    """With s_q = s_kv the last row sees every key under both masks (codelab step 7)."""
    rng = np.random.default_rng(3)
    q, k, v = (_rand(rng, 2, 3, 16, 4) for _ in range(3))
    oc, lc = attention_forward(q, k, v, 0.5, True)
    on, ln = attention_forward(q, k, v, 0.5, False)
    np.testing.assert_allclose(oc[:, :, -1], on[:, :, -1], atol=1e-14)
    np.testing.assert_allclose(lc[:, :, -1], ln[:, :, -1], atol=1e-14)
    assert np.abs(oc[:, :, 0] - on[:, :, 0]).max() > 0.1


@pytest.mark.parametrize("which", ["q", "k"])
def test_zero_scores_give_column_means(which):
    """Q = 0 (or K = 0): uniform weights, O_i = mean of visible V rows, LSE_i = ln(#visible)."""
    rng = np.random.default_rng(4)
    s, d = 10, 6
    q, k, v = _rand(rng, 1, 2, s, d), _rand(rng, 1, 2, s, d), _rand(rng, 1, 2, s, d)
    if which == "q":
        q[:] = 0
    else:
        k[:] = 0
    o, l = attention_forward(q, k, v, 0.7, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_allclose(l, math.log(s), atol=1e-14)
    oc, lc = attention_forward(q, k, v, 0.7, True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, s + 1)[None, None, :, None]
    np.testing.assert_allclose(oc, prefix, atol=1e-14)
    np.testing.assert_allclose(lc, np.broadcast_to(np.log(np.arange(1, s + 1)), lc.shape), atol=1e-14)


def test_row_shift_invariance():
    """K_j -> K_j + c shifts row i's scores by scale*q_i.c: O unchanged, LSE_i += scale*q_i.c."""
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4)
    c = _rand(rng, 4) * 3
    scale = 0.45
    for causal in (False, True):
        o1, l1 = attention_forward(q, k, v, scale, causal)
        o2, l2 = attention_forward(q, k + c, v, scale, causal)
        np.testing.assert_allclose(o2, o1, atol=1e-12)
        np.testing.assert_allclose(l2, l1 + scale * (q @ c), atol=1e-12)


def test_gqa_equals_repeated_mha():
    """Each KV head serves a contiguous group of query heads (codelab step 9)."""
    rng = np.random.default_rng(6)
    h_q, h_kv = 8, 2
    q, do = _rand(rng, 2, h_q, 7, 4), _rand(rng, 2, h_q, 7, 4)
    k, v = _rand(rng, 2, h_kv, 7, 4), _rand(rng, 2, h_kv, 7, 4)
    kr, vr = np.repeat(k, h_q // h_kv, axis=1), np.repeat(v, h_q // h_kv, axis=1)
    for causal in (False, True):
        o1, l1 = attention_forward(q, k, v, 0.3, causal)
        o2, l2 = attention_forward(q, kr, vr, 0.3, causal)
        np.testing.assert_allclose(o1, o2, atol=1e-14)
        np.testing.assert_allclose(l1, l2, atol=1e-14)
        dq1, dk1, dv1 = attention_backward(q, k, v, do, 0.3, causal)
        dq2, dk2, dv2 = attention_backward(q, kr, vr, do, 0.3, causal)
        np.testing.assert_allclose(dq1, dq2, atol=1e-13)
        np.testing.assert_allclose(dk1, dk2.reshape(2, h_kv, 4, 7, 4).sum(2), atol=1e-13)
        np.testing.assert_allclose(dv1, dv2.reshape(2, h_kv, 4, 7, 4).sum(2), atol=1e-13)


def test_constant_v_and_key_gradient_sum():
    """V rows all equal c: O = c and dQ = dK = 0. For any V: sum_j dK_j = 0 (rows of dS sum to 0)."""
    rng = np.random.default_rng(7)
    q, k, do = _rand(rng, 1, 2, 8, 3), _rand(rng, 1, 1, 8, 3), _rand(rng, 1, 2, 8, 3)
    c = np.array([0.5, -2.0, 1.25])
    v = np.broadcast_to(c, (1, 1, 8, 3)).copy()
    for causal in (False, True):
        o, _ = attention_forward(q, k, v, 0.6, causal)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-14)
        dq, dk, dv = attention_backward(q, k, v, do, 0.6, causal)
        np.testing.assert_allclose(dq, 0, atol=1e-13)
        np.testing.assert_allclose(dk, 0, atol=1e-13)
        v2 = _rand(rng, 1, 1, 8, 3)
        _, dk2, _ = attention_backward(q, k, v2, do, 0.6, causal)
        np.testing.assert_allclose(dk2.sum(axis=2), 0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(2, 2), (2, 1)])
def test_backward_matches_finite_differences(causal, heads):
    """Central differences of L = sum(O * dO), eps = 1e-6, in float64."""
    h_q, h_kv = heads
    rng = np.random.default_rng(8 + causal)
    s_q, s_kv, d = 5, 6, 3
    q, k, v = _rand(rng, 1, h_q, s_q, d), _rand(rng, 1, h_kv, s_kv, d), _rand(rng, 1, h_kv, s_kv, d)
    do = _rand(rng, 1, h_q, s_q, d)
    scale = 0.8

    def loss(q_, k_, v_):
        return float((attention_forward(q_, k_, v_, scale, causal)[0] * do).sum())

    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v, name: xp}
            args_m = {"q": q, "k": k, "v": v, name: xm}
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"])
                        - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        err = np.abs(num - g).max() / max(1e-12, np.abs(g).max())
        assert err < 1e-6, (name, err)


# --------------------------------------------------------------------------
# Library routine: torch's SDPA in float64 on the CPU (the "Using cuDNN in
# Python" page checks its output against the same routine).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(4, 4), (4, 2), (4, 1)])
def test_against_torch_sdpa_float64(causal, heads):
    h_q, h_kv = heads
    rng = np.random.default_rng(10 + h_kv)
    b, s, d = 2, 33, 16
    q, k, v, do = _rand(rng, b, h_q, s, d), _rand(rng, b, h_kv, s, d), _rand(rng, b, h_kv, s, d), \
        _rand(rng, b, h_q, s, d)
    scale = 1 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                                          enable_gqa=(h_q != h_kv))
    (to * torch.tensor(do)).sum().backward()
    o, _ = attention_forward(q, k, v, scale, causal, row_block=10)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal, row_block=10)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_subsets_equal_full():
    """heads/rows/kv_heads subsets give the same values as the full computation."""
    rng = np.random.default_rng(11)
    q, k, v, do = _rand(rng, 2, 4, 20, 4), _rand(rng, 2, 2, 20, 4), _rand(rng, 2, 2, 20, 4), \
        _rand(rng, 2, 4, 20, 4)
    o, l = attention_forward(q, k, v, 0.5, True)
    rows = np.array([0, 7, 19])
    os_, ls_ = attention_forward(q, k, v, 0.5, True, heads=[(1, 3)], rows=rows)
    np.testing.assert_array_equal(os_[1, 3], o[1, 3, rows])
    np.testing.assert_array_equal(ls_[1, 3], l[1, 3, rows])
    assert np.isnan(os_[0, 0]).all()
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, True)
    dqs, dks, dvs = attention_backward(q, k, v, do, 0.5, True, kv_heads=[(0, 1)])
    np.testing.assert_array_equal(dks[0, 1], dk[0, 1])
    np.testing.assert_array_equal(dqs[0, 2:4], dq[0, 2:4])


# --------------------------------------------------------------------------
# FP8 e4m3 decoding (JAX attention codelab, step 10: E4M3 in the forward).
# --------------------------------------------------------------------------
def test_fp8_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8_e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert fp8_e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert fp8_e4m3_decode(np.array([0x38]))[0] == 1.0
    assert fp8_e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9


def test_fp8_e5m2_decode_matches_torch_for_all_codes():
    """E5M2 (the HYBRID format's gradient type, codelab step 10) against torch's
    float8_e5m2 for every code, plus the values the format's definition fixes."""
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8_e5m2_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 6  # exponent 31 with a nonzero mantissa, both signs
    assert (np.isnan(ours) == nan).all()
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert fp8_e5m2_decode(np.array([0x7B]))[0] == 57344.0
    assert fp8_e5m2_decode(np.array([0x3C]))[0] == 1.0
    assert fp8_e5m2_decode(np.array([0x01]))[0] == 2.0 ** -16
    assert fp8_e5m2_decode(np.array([0x7C]))[0] == np.inf
    assert fp8_e5m2_decode(np.array([0xFC]))[0] == -np.inf
    # e5m2 is the upper byte of an IEEE half: same value for every code
    half = (codes.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(ours[~nan], half[~nan])
    assert fp8_dequantize(np.array([0x3C], dtype=np.uint8), 0.25, "e5m2")[0] == 0.25


def test_fp8_e5m2_gradient_roundtrip():
    """dO of an fp8 backward workload is e5m2 with its descale; it dequantises to
    within e5m2's half-ulp (relative 2^-3) of the drawn values."""
    w = sdpa_inputs.Workload("t", 1, 2, 2, 64, 64, 32, "fp8", "bf16", False, 0.2, "bshd", 5, backward=True)
    ins = sdpa_inputs.make_inputs(w)
    assert ins["do"].dtype == torch.float8_e5m2
    deq = fp8_dequantize(ins["do"].view(torch.uint8).numpy(), ins["descale_do"], "e5m2")
    gen = torch.Generator().manual_seed(5)
    for _ in range(3):
        sdpa_inputs.randn_logical(gen, 1, 2, 64, 32, "bshd", "f32")
    do32 = sdpa_inputs.randn_logical(gen, 1, 2, 64, 32, "bshd", "f32").numpy()
    amax = np.abs(do32).max()
    assert np.abs(deq).max() == pytest.approx(amax, rel=1e-6)
    big = np.abs(do32) > amax * 2 ** -10
    assert (np.abs(deq - do32)[big] <= np.abs(do32)[big] * 2 ** -3 * 1.0001).all()


def test_fp8_inputs_roundtrip():
    """Quantised inputs dequantise to within e4m3's half-ulp of the drawn values."""
    w = sdpa_inputs.Workload("t", 1, 2, 2, 64, 64, 32, "fp8", "bf16", False, 0.2, "bshd", 5)
    ins = sdpa_inputs.make_inputs(w)
    gen = torch.Generator().manual_seed(5)
    q32 = sdpa_inputs.randn_logical(gen, 1, 2, 64, 32, "bshd", "f32").numpy()
    deq = fp8_dequantize(ins["q"].view(torch.uint8).numpy(), ins["descale_q"])
    amax = np.abs(q32).max()
    assert np.abs(deq).max() == pytest.approx(amax, rel=1e-6)
    # relative error of e4m3 for normal values is <= 2^-4
    big = np.abs(q32) > amax * 2 ** -5
    assert (np.abs(deq - q32)[big] <= np.abs(q32)[big] * 2 ** -4 * 1.0001).all()


# --------------------------------------------------------------------------
# What the pages print for their worked examples.
# --------------------------------------------------------------------------
def test_pages_printed_shapes_and_layouts():
    g = json.load(open(GOLDEN))
    rng = np.random.default_rng(12)
    # step 3/4 of the codelab: output has Q's shape (B, T, N, H)
    B, T, N, H = g["naive_output_shape"]["input_bthn"]
    q = _rand(rng, B, T, N, H)
    qb = q.transpose(0, 2, 1, 3)[:, :, :8]  # a few rows suffice for the shape
    o, _ = attention_forward(qb, qb, qb, 1 / math.sqrt(H), False)
    assert o.transpose(0, 2, 1, 3).shape == (B, 8, N, H)
    # step 9: MHA / GQA / MQA keep the output shape
    Bq, Tq, Nq, Hq = g["head_variants"]["q_bthn"]
    qh = _rand(rng, Bq, Nq, Tq, Hq)
    for nk in g["head_variants"]["kv_heads"]:
        kh = _rand(rng, Bq, nk, Tq, Hq)
        o, _ = attention_forward(qh, kh, kh, 0.125, False)
        assert list(o.transpose(0, 2, 1, 3).shape) == g["head_variants"]["output_bthn"]
    # "Using cuDNN in Python": BSHD strides and scale
    c = g["gpt2_bshd"]
    assert sdpa_inputs.logical_strides(c["b"], c["h"], c["s"], c["d"], "bshd") == tuple(c["bshd_strides"])
    assert sdpa_inputs.gpt2().scale == c["attn_scale"] == 1 / math.sqrt(c["d"])
    x = sdpa_inputs.randn_logical(torch.Generator().manual_seed(0), 2, 3, 4, 8, "bshd", "f32")
    assert x.stride() == sdpa_inputs.logical_strides(2, 3, 4, 8, "bshd")


def test_inputs_same_bits_for_both_sides():
    """The generator is deterministic per seed and rounds to the I/O dtype once."""
    w = sdpa_inputs.hd128(512)
    w.b = 1
    a = sdpa_inputs.make_inputs(w)
    b = sdpa_inputs.make_inputs(w)
    for name in ("q", "k", "v", "do"):
        assert a[name].dtype == torch.bfloat16
        assert torch.equal(a[name].view(torch.int16), b[name].view(torch.int16))
        assert a[name].stride() == sdpa_inputs.logical_strides(1, 16, 512, 128, "bshd")
