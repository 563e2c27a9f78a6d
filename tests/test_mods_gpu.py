"""GPU parity of the score modifiers (additive bias tensor, ALiBi) against the
float64 oracle: forward (bf16, f16, f32) and backward (bf16, f16), with the
bias broadcast over batch and/or heads, in fp32 or the io dtype, together
with the causal masks and padding lengths."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from oracle import attention_backward, attention_forward
from sdpa_inputs import Workload
from tests.parity import LSE_REL, TOL, check_out, f64, say, to_gpu

pytestmark = pytest.mark.gpu

ALIGN = {"none": (False, "top_left"), "causal": (True, "top_left"), "bottom_right": (True, "bottom_right")}
CAUSAL_ARG = {"none": False, "causal": True, "bottom_right": "bottom_right"}


def _mods(w, bias_shape, bias_dtype, alibi, seed):
    bias = None if bias_shape is None else sdpa_inputs.make_bias(bias_shape + (w.s_q, w.s_kv), seed, bias_dtype)
    slopes = sdpa.alibi_slopes(w.h_q, device="cpu") if alibi else None
    return bias, slopes


def _oracle_kw(bias, slopes):
    return dict(bias=None if bias is None else bias.double().numpy(),
                alibi_slopes=None if slopes is None else slopes.double().numpy())


def _gpu_kw(bias, slopes):
    return dict(bias=None if bias is None else bias.cuda(), alibi_slopes=None if slopes is None else slopes.cuda())


def _check_lse(lg, lr):
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr))
    fin = np.isfinite(lr)
    err = np.abs(lg[fin] - lr[fin]) / np.maximum(1.0, np.abs(lr[fin]))
    assert err.max() <= LSE_REL, err.max()


@pytest.mark.parametrize("mods", [((2, 4), "f32", False), ((1, 4), "io", True), ((1, 1), "io", False),
                                  (None, None, True), ((2, 1), "f32", True)])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fwd_score_modifiers(dtype, d, mask, mods):
    bias_shape, bias_dt, alibi = mods
    if dtype == "f32" and bias_dt == "io":
        bias_dt = "f32"
    w = Workload("fwd_mod", 2, 4, 2, 200, 232, d, dtype, dtype, mask != "none", 1 / math.sqrt(d), "bshd", 600 + d)
    bias, slopes = _mods(w, bias_shape, dtype if bias_dt == "io" else bias_dt, alibi, w.seed + 1)
    say(f"[mods fwd] {w} mask={mask} bias={bias_shape}/{bias_dt} alibi={alibi}")
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=CAUSAL_ARG[mask], **_gpu_kw(bias, slopes))
    torch.cuda.synchronize()
    causal, align = ALIGN[mask]
    q, k, v = (f64(ins[n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = attention_forward(q, k, v, w.scale, causal, align=align, **_oracle_kw(bias, slopes))
    check_out(f64(o.cpu()), o_ref, TOL[w.out_dtype], what="O: ")
    _check_lse(lse.cpu().numpy(), lse_ref)


def _fwd_bwd(w, g, mask, kw, lq=None, lk=None):
    lens = dict(seq_len_q=None if lq is None else lq.cuda(), seq_len_kv=None if lk is None else lk.cuda())
    o, lse = sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=CAUSAL_ARG[mask], **kw, **lens)
    grads = sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=CAUSAL_ARG[mask], **kw, **lens)
    torch.cuda.synchronize()
    return o, lse, grads


def _check_grads(w, grads, refs):
    tol = 2 * TOL[w.out_dtype]
    for name, x, r in zip(("dq", "dk", "dv"), grads, refs):
        check_out(f64(x.cpu()), r, tol, grad_dtype=w.out_dtype, what=f"{name}: ")


@pytest.mark.parametrize("mods", [((1, 4), "f32", True), ((2, 4), "io", False), (None, None, True)])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bwd_score_modifiers(dtype, d, mask, mods):
    bias_shape, bias_dt, alibi = mods
    w = Workload("bwd_mod", 2, 4, 2, 296, 296, d, dtype, dtype, mask != "none", 1 / math.sqrt(d), "bshd",
                 700 + d, backward=True)
    bias, slopes = _mods(w, bias_shape, dtype if bias_dt == "io" else bias_dt, alibi, w.seed + 1)
    say(f"[mods bwd] {w} mask={mask} bias={bias_shape}/{bias_dt} alibi={alibi}")
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    _, _, grads = _fwd_bwd(w, g, mask, _gpu_kw(bias, slopes))
    causal, align = ALIGN[mask]
    q, k, v, do = (f64(ins[n]) for n in ("q", "k", "v", "do"))
    _check_grads(w, grads, attention_backward(q, k, v, do, w.scale, causal, align=align, **_oracle_kw(bias, slopes)))


@pytest.mark.parametrize("h_kv", [8, 1])
def test_mods_with_padding_bottom_right_gqa(h_kv):
    """ALiBi + bias with padding lengths and the bottom-right diagonal (the
    ALiBi distance uses the same offset), GQA/MQA (split-group dK/dV path)."""
    w = Workload("mods_pad", 2, 8, h_kv, 190, 264, 128, "bf16", "bf16", True, 1 / math.sqrt(128), "bhsd",
                 800 + h_kv, backward=True)
    lq, lk = torch.tensor([190, 77], dtype=torch.int32), torch.tensor([150, 264], dtype=torch.int32)
    bias, slopes = _mods(w, (1, 8), "bf16", True, w.seed + 1)
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    o, lse, grads = _fwd_bwd(w, g, "bottom_right", _gpu_kw(bias, slopes), lq, lk)
    q, k, v, do = (f64(ins[n]) for n in ("q", "k", "v", "do"))
    kw = dict(seq_len_q=lq.numpy(), seq_len_kv=lk.numpy(), align="bottom_right", **_oracle_kw(bias, slopes))
    o_ref, lse_ref = attention_forward(q, k, v, w.scale, True, **kw)
    check_out(f64(o.cpu()), o_ref, TOL["bf16"], what="O: ")
    _check_lse(lse.cpu().numpy(), lse_ref)
    _check_grads(w, grads, attention_backward(q, k, v, do, w.scale, True, **kw))


def test_mods_rejected_for_fp8():
    w = sdpa_inputs.Workload("fp8_mod", 1, 2, 2, 64, 64, 128, "fp8", "bf16", False, 1 / math.sqrt(128), "bshd", 1)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    sc = sdpa.Fp8Scales(ins["descale_q"], ins["descale_k"], ins["descale_v"], ins["scale_p"], ins["descale_p"])
    with pytest.raises(sdpa.SdpaError, match="not supported with fp8"):
        sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, fp8=sc, alibi_slopes=sdpa.alibi_slopes(2))
