"""GPU parity of dropout (Philox4x32-10 mask regenerated in the backward)
against the float64 oracle, which builds the same mask from the same rule:
the keep decisions are integer comparisons of the same random bytes, so any
mismatch shows as an error far beyond the tolerance."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from oracle import attention_backward, attention_forward
from sdpa_inputs import Workload
from tests.parity import LSE_REL, TOL, excess_err, f64, max_abs, say, to_gpu

pytestmark = pytest.mark.gpu

CAUSAL_ARG = {"none": False, "causal": True, "bottom_right": "bottom_right"}
ALIGN = {"none": (False, "top_left"), "causal": (True, "top_left"), "bottom_right": (True, "bottom_right")}


def _drop(p, seed, offset):
    # the ABI carries p as fp32; the oracle gets the same value
    return dict(dropout_p=float(np.float32(p)), dropout_seed=seed, dropout_offset=offset)


def _run(w, g, mask, drop, backward, **extra):
    o, lse = sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=CAUSAL_ARG[mask], **drop, **extra)
    grads = None
    if backward:
        grads = sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=CAUSAL_ARG[mask], **drop,
                         **extra)
    torch.cuda.synchronize()
    return o, lse, grads


def _check_o(w, o, o_ref):
    og = f64(o.cpu())
    exc = excess_err(og, o_ref, w.out_dtype)
    say(f"    O: max|err|={max_abs(og, o_ref):.3e} beyond-rounding={exc:.3e}")
    assert exc <= TOL[w.out_dtype], exc


def _check_lse(lg, lr):
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr))
    fin = np.isfinite(lr)
    err = np.abs(lg[fin] - lr[fin]) / np.maximum(1.0, np.abs(lr[fin]))
    assert err.max() <= LSE_REL


def _check_grads(w, grads, refs):
    for name, x, r in zip(("dq", "dk", "dv"), grads, refs):
        xa = f64(x.cpu())
        exc = excess_err(xa, r, w.out_dtype)
        say(f"    {name}: max|err|={max_abs(xa, r):.3e} beyond-rounding={exc:.3e} max|ref|={np.abs(r).max():.2f}")
        assert exc <= 2 * TOL[w.out_dtype], (name, exc)


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_dropout_fwd_bwd(dtype, d, mask, p):
    w = Workload("drop", 2, 4, 2, 290, 290, d, dtype, dtype, mask != "none", 1 / math.sqrt(d), "bshd",
                 900 + d, backward=True)
    drop = _drop(p, 0x5EED0000 + d, 3)
    say(f"[dropout] {w} mask={mask} {drop}")
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    o, lse, grads = _run(w, g, mask, drop, True)
    causal, align = ALIGN[mask]
    q, k, v, do = (f64(ins[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = attention_forward(q, k, v, w.scale, causal, align=align, **drop)
    _check_o(w, o, o_ref)
    _check_lse(lse.cpu().numpy(), lse_ref)
    _check_grads(w, grads, attention_backward(q, k, v, do, w.scale, causal, align=align, **drop))


@pytest.mark.parametrize("h_kv", [8, 1])
def test_dropout_with_alibi_padding_gqa(h_kv):
    w = Workload("drop_mix", 2, 8, h_kv, 200, 264, 128, "bf16", "bf16", True, 1 / math.sqrt(128), "bhsd",
                 950 + h_kv, backward=True)
    lq, lk = torch.tensor([200, 90], dtype=torch.int32), torch.tensor([170, 264], dtype=torch.int32)
    drop = _drop(0.25, 1234567890123, 41)
    slopes = sdpa.alibi_slopes(w.h_q, device="cpu")
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    o, lse, grads = _run(w, g, "bottom_right", drop, True, seq_len_q=lq.cuda(), seq_len_kv=lk.cuda(),
                         alibi_slopes=slopes.cuda())
    q, k, v, do = (f64(ins[n]) for n in ("q", "k", "v", "do"))
    kw = dict(seq_len_q=lq.numpy(), seq_len_kv=lk.numpy(), align="bottom_right",
              alibi_slopes=slopes.double().numpy(), **drop)
    o_ref, lse_ref = attention_forward(q, k, v, w.scale, True, **kw)
    _check_o(w, o, o_ref)
    _check_lse(lse.cpu().numpy(), lse_ref)
    _check_grads(w, grads, attention_backward(q, k, v, do, w.scale, True, **kw))


def test_dropout_all_and_none():
    w = Workload("drop_lim", 1, 2, 2, 100, 100, 64, "f16", "f16", False, 0.125, "bshd", 7, backward=True)
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    o, lse, grads = _run(w, g, "none", _drop(1.0, 5, 0), True)
    assert (o == 0).all() and all((x == 0).all() for x in grads)
    o0, lse0, _ = _run(w, g, "none", {}, False)
    o1, lse1, _ = _run(w, g, "none", _drop(0.0, 5, 0), False)
    assert torch.equal(o0, o1) and torch.equal(lse0, lse1)
    # LSE is that of the undropped weights; the modifier kernel scales the
    # scores before the row max, so it agrees within rounding, not bitwise
    torch.testing.assert_close(lse, lse0, rtol=1e-6, atol=1e-6)


def test_dropout_deterministic_and_offset_dependent():
    w = Workload("drop_det", 1, 4, 4, 256, 256, 128, "bf16", "bf16", True, 1 / math.sqrt(128), "bshd", 8)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    a, _, _ = _run(w, g, "causal", _drop(0.3, 99, 1), False)
    b, _, _ = _run(w, g, "causal", _drop(0.3, 99, 1), False)
    c, _, _ = _run(w, g, "causal", _drop(0.3, 99, 2), False)
    assert torch.equal(a, b) and not torch.equal(a, c)


def test_dropout_rejected_for_f32():
    w = Workload("drop_f32", 1, 2, 2, 64, 64, 64, "f32", "f32", False, 0.125, "bhsd", 1)
    g = to_gpu(sdpa_inputs.make_inputs(w))
    with pytest.raises(sdpa.SdpaError, match="dropout needs"):
        sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, dropout_p=0.1)
