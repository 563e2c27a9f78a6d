"""GPU parity of the fp8 backward (HYBRID format of the JAX attention codelab,
step 10: q, k, v in e4m3, the gradient dO in e5m2) against the float64 oracle.

The oracle takes the dequantised tensors (code x per-tensor descale) and
computes the exact gradients, including its own exact O. The kernel widens the
codes exactly and runs the 16-bit backward with the descales folded in, so its
own rounding matches the bf16 backward's; what the fp8 tolerance absorbs is the
O it is handed: the fp8 forward quantises P to e4m3, and D = rowsum(dO * O)
inherits that error. Checks per gradient: max-abs error beyond bf16 rounding
<= 2 x 1e-1 (twice the fp8 forward's, as for every gradient) and a relative
Frobenius error <= 1e-1. With O and LSE from the oracle itself the kernel
sees exact statistics, and the bf16 gradient bound 2 x 2e-2 applies."""
import math

import pytest
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from oracle import attention_forward
from sdpa_inputs import Workload
from tests.parity import TOL, check_out, f64, oracle_bwd, rel_fro, say, to_gpu

pytestmark = pytest.mark.gpu


def _fp8_fwd(w, g, causal, lq=None, lk=None):
    fp8 = sdpa.Fp8Scales(g["descale_q"], g["descale_k"], g["descale_v"], g["scale_p"], g["descale_p"])
    o, lse = sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=causal, fp8=fp8, seq_len_q=lq,
                      seq_len_kv=lk)
    return o, lse


def _fp8_bwd(w, g, o, lse, causal, lq=None, lk=None):
    dq, dk, dv = sdpa.bwd_fp8(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=causal,
                              descale_q=g["descale_q"], descale_k=g["descale_k"], descale_v=g["descale_v"],
                              descale_do=g["descale_do"], seq_len_q=lq, seq_len_kv=lk)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check(grads, refs, tol, rf_tol, tag=""):
    for name, x, r in zip(("dq", "dk", "dv"), grads, refs):
        assert x.dtype == torch.bfloat16
        xa = f64(x.cpu())
        check_out(xa, r, tol, grad_dtype="bf16", what=f"{tag}{name}: ")
        rf = rel_fro(xa, r)
        assert rf <= rf_tol, (name, rf)


def _run(w, causal=None, lens=None, seed=0):
    causal = w.causal if causal is None else causal
    say(f"[fp8 bwd] {w} causal={causal} lens={lens is not None}")
    ins = sdpa_inputs.make_inputs(w)
    assert ins["do"].dtype == torch.float8_e5m2
    g = to_gpu(ins)
    lq = lk = None
    if lens is not None:
        lq = sdpa_inputs.make_lengths(w.b, w.s_q, seed, min_len=lens)
        lk = sdpa_inputs.make_lengths(w.b, w.s_kv, seed + 1, min_len=lens)
    lqg = None if lq is None else lq.cuda()
    lkg = None if lk is None else lk.cuda()
    o, lse = _fp8_fwd(w, g, causal, lqg, lkg)
    grads = _fp8_bwd(w, g, o, lse, causal, lqg, lkg)
    align = "bottom_right" if causal == "bottom_right" else "top_left"
    refs = oracle_bwd(w, ins, seq_len_q=None if lq is None else lq.numpy(),
                      seq_len_kv=None if lk is None else lk.numpy(), align=align)
    _check(grads, refs, 2 * TOL["fp8"], TOL["fp8"])
    return ins, g, grads


def _fp8_workload(name, b, h_q, h_kv, s_q, s_kv, d, causal, layout, seed):
    return Workload(name, b, h_q, h_kv, s_q, s_kv, d, "fp8", "bf16", causal, 1 / math.sqrt(d), layout, seed,
                    backward=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_bwd_small(causal):
    _run(_fp8_workload("fp8_bwd", 2, 4, 4, 300, 300, 128, causal, "bshd", 31))


@pytest.mark.parametrize("h_kv", [2, 1])
def test_fp8_bwd_gqa_ragged(h_kv):
    """GQA / MQA, unequal ragged lengths, BHSD strides, top-left causal."""
    _run(_fp8_workload("fp8_bwd_gqa", 1, 8, h_kv, 161, 230, 128, True, "bhsd", 5 + h_kv))


def test_fp8_bwd_padding_bottom_right():
    """Per-batch valid lengths and the bottom-right diagonal."""
    _run(_fp8_workload("fp8_bwd_pad", 3, 4, 2, 200, 264, 128, True, "bshd", 77), causal="bottom_right",
         lens=16, seed=9)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_bwd_d64_exact_statistics(causal):
    """d = 64 (no fp8 forward at this width): O and LSE from the oracle's forward
    (O rounded to bf16), so only the backward's own rounding remains."""
    w = _fp8_workload("fp8_bwd_d64", 2, 4, 2, 257, 257, 64, causal, "bshd", 64)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    q, k, v = (f64(ins[n], ins["descale_" + n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = attention_forward(q, k, v, w.scale, causal)
    o = sdpa_inputs.to_device_like(torch.from_numpy(o_ref).to(torch.bfloat16), "cuda")
    lse = torch.from_numpy(lse_ref).float().contiguous().cuda()
    grads = _fp8_bwd(w, g, o, lse, causal)
    _check(grads, oracle_bwd(w, ins), 2 * TOL["bf16"], 2 * TOL["bf16"])


def test_fp8_bwd_e4m3_gradient():
    """dO given in e4m3 instead of e5m2 (the all-E4M3 recipe)."""
    w = _fp8_workload("fp8_bwd_e4m3do", 1, 4, 4, 190, 190, 128, True, "bshd", 12)
    ins = sdpa_inputs.make_inputs(w)
    do32 = f64(ins["do"], ins["descale_do"])
    ins["do"], ins["descale_do"] = sdpa_inputs.quantize_fp8(torch.from_numpy(do32).float(), "e4m3")
    g = to_gpu(ins)
    o, lse = _fp8_fwd(w, g, True)
    grads = _fp8_bwd(w, g, o, lse, True)
    _check(grads, oracle_bwd(w, ins), 2 * TOL["fp8"], TOL["fp8"])


def test_fp8_bwd_matches_scaled_codes():
    """Descale factors fold in exactly: doubling dO's descale (a power of two,
    exact in fp32) doubles all three gradients bit for bit, since each is
    linear in dO and the factor only enters their output scales."""
    w = _fp8_workload("fp8_bwd_fold", 1, 2, 2, 130, 130, 128, True, "bshd", 3)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = _fp8_fwd(w, g, True)
    base = _fp8_bwd(w, g, o, lse, True)
    g2 = dict(g, descale_do=g["descale_do"] * 2)
    twice = _fp8_bwd(w, g2, o, lse, True)
    for x, y in zip(base, twice):
        torch.testing.assert_close(y.float(), 2 * x.float(), rtol=0, atol=0)


def test_fp8_bwd_no_query_rows_zeroes_dkdv():
    w = _fp8_workload("fp8_bwd_empty", 1, 2, 2, 0, 64, 128, False, "bshd", 1)
    k = torch.zeros(1, 64, 2, 128, device="cuda").to(torch.float8_e4m3fn).permute(0, 2, 1, 3)
    q = torch.zeros(1, 0, 2, 128, device="cuda").to(torch.float8_e4m3fn).permute(0, 2, 1, 3)
    do = torch.zeros(1, 0, 2, 128, device="cuda").to(torch.float8_e5m2).permute(0, 2, 1, 3)
    o = torch.zeros(1, 0, 2, 128, device="cuda", dtype=torch.bfloat16).permute(0, 2, 1, 3)
    lse = torch.zeros(1, 2, 0, device="cuda")
    dk = torch.full((1, 64, 2, 128), 7.0, device="cuda", dtype=torch.bfloat16).permute(0, 2, 1, 3)
    dv = torch.full_like(dk, 7.0)
    sdpa.bwd_fp8(q, k, k, o, do, lse, scale=w.scale, descale_q=1.0, descale_k=1.0, descale_v=1.0,
                 descale_do=1.0, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert dk.abs().max().item() == 0 and dv.abs().max().item() == 0


def test_fp8_bwd_full_size_sampled():
    """b2 h16 s8192 d128 causal (the hd128 training shape) in fp8: one KV head's gradients."""
    w = sdpa_inputs.fp8_hd128()
    say(f"[fp8 bwd sampled] {w}")
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = _fp8_fwd(w, g, True)
    grads = _fp8_bwd(w, g, o, lse, True)
    groups = [(w.b - 1, w.h_kv - 1)]
    refs = oracle_bwd(w, ins, kv_heads=groups)
    _check(grads, refs, 2 * TOL["fp8"], TOL["fp8"], tag=f"groups={groups} ")
