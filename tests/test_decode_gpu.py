"""GPU parity of the split-KV forward (few query rows against a long key
range: a KV-cache step) against the float64 oracle.

The split-KV path groups the query heads of a KV head into shared row blocks
and merges per-split partials; the oracle is the plain row softmax. Checks:
O max-abs beyond output rounding within the dtype's tolerance, LSE within
1e-3 relative, rows that see no key O = 0 / LSE = -inf; and agreement with the
row-block kernel on the same inputs (the same values, associated differently)."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from oracle import attention_forward
from sdpa_inputs import Workload
from tests.parity import LSE_REL, TOL, check_out, f64, say, to_gpu

pytestmark = pytest.mark.gpu


def _oracle(w, ins, mask, lq, lk, heads=None):
    causal, align = {"none": (False, "top_left"), "causal": (True, "top_left"),
                     "bottom_right": (True, "bottom_right")}[mask]
    q, k, v = (f64(ins[n]) for n in ("q", "k", "v"))
    return attention_forward(q, k, v, w.scale, causal, heads=heads,
                             seq_len_q=None if lq is None else lq.numpy(),
                             seq_len_kv=None if lk is None else lk.numpy(), align=align)


def _run(w, g, mask, lq, lk, split_kv=True):
    causal = {"none": False, "causal": True, "bottom_right": "bottom_right"}[mask]
    o, lse = sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=causal, split_kv=split_kv,
                      seq_len_q=None if lq is None else lq.cuda(), seq_len_kv=None if lk is None else lk.cuda())
    torch.cuda.synchronize()
    return o, lse


def _check(w, o, lse, o_ref, lse_ref, heads=None):
    og, lg = f64(o.cpu()), lse.cpu().numpy()
    if heads is not None:
        sel = np.zeros(og.shape[:2], dtype=bool)
        for bi, hq in heads:
            sel[bi, hq] = True
        og, lg, o_ref, lse_ref = og[sel], lg[sel], o_ref[sel], lse_ref[sel]
    check_out(og, o_ref, TOL[w.out_dtype], what="O: ")
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty)
    assert (og[empty] == 0).all()
    fin = np.isfinite(lse_ref)
    if fin.any():
        err = np.abs(lg[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        assert err.max() <= LSE_REL, err.max()


@pytest.mark.parametrize("mask", ["none", "bottom_right", "causal"])
@pytest.mark.parametrize("s_q", [1, 3, 16])
@pytest.mark.parametrize("heads", [(32, 8), (32, 1), (8, 8)])
def test_split_kv_bf16_d128(heads, s_q, mask):
    h_q, h_kv = heads
    w = Workload("decode", 2, h_q, h_kv, s_q, 5000, 128, "bf16", "bf16", mask != "none", 1 / math.sqrt(128),
                 "bshd", 500 + s_q + h_kv)
    assert sdpa.fwd_workspace_size(w.b, h_q, h_kv, s_q, w.s_kv, 128, torch.bfloat16) > 0
    lk = torch.tensor([5000, 3333], dtype=torch.int32)
    say(f"[decode] {w} mask={mask}")
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = _run(w, g, mask, None, lk)
    o_ref, lse_ref = _oracle(w, ins, mask, None, lk)
    _check(w, o, lse, o_ref, lse_ref)
    # the row-block kernel on the same inputs agrees within rounding
    o2, lse2 = _run(w, g, mask, None, lk, split_kv=False)
    _check(w, o2, lse2, o_ref, lse_ref)


@pytest.mark.parametrize("s_kv", [777, 4099])
def test_split_kv_f16_d64_padded_queries(s_kv):
    w = Workload("decode64", 3, 16, 4, 5, s_kv, 64, "f16", "f16", True, 0.125, "bhsd", 7 + s_kv)
    lq = torch.tensor([5, 2, 0], dtype=torch.int32)
    lk = torch.tensor([s_kv, s_kv // 2, 100], dtype=torch.int32)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = _run(w, g, "bottom_right", lq, lk)
    o_ref, lse_ref = _oracle(w, ins, "bottom_right", lq, lk)
    _check(w, o, lse, o_ref, lse_ref)


def test_split_kv_kv_cache_full_size_sampled():
    """b8 h_q32 h_kv8 one new token against a 32768-key cache (1 GiB of K/V),
    bottom-right causal with per-batch cache lengths; sampled heads."""
    w = Workload("decode_full", 8, 32, 8, 1, 32768, 128, "bf16", "bf16", True, 1 / math.sqrt(128), "bshd", 32768)
    lk = sdpa_inputs.make_lengths(w.b, w.s_kv, w.seed, min_len=1)
    say(f"[decode full] {w} lk={lk.tolist()}")
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = _run(w, g, "bottom_right", None, lk)
    heads = [(0, 0), (1, 5), (3, 31), (7, 12), (5, 20)]
    o_ref, lse_ref = _oracle(w, ins, "bottom_right", None, lk, heads=heads)
    _check(w, o, lse, o_ref, lse_ref, heads=heads)
