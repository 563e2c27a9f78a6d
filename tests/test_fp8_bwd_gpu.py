"""GPU parity of the fp8 backward (HYBRID format of the JAX attention codelab,
step 10: q, k, v in e4m3, the gradient dO in e5m2) against the float64 oracle.

The oracle takes the dequantised tensors (code x per-tensor descale) and
computes the exact gradients, including its own exact O. The kernel runs all
five products on fp8 operands: P enters dV as e4m3 (P x 448) and dS enters dK
and dQ as e4m3 (the default) or e5m2, with scale_ds chosen as the recipe's
delayed scaling would (the power of two that maps max |dS| just inside the
format); it also gets the fp8 forward's O (P quantised to e4m3), which D =
rowsum(dO * O) inherits. Bounds per gradient:
- dS in e4m3: max-abs error <= 2 x 1e-1 (twice the fp8 forward's, as for every
  gradient; bf16 rounding slack only where bf16's half-ulp reaches half the
  bound) and relative Frobenius error <= 1e-1;
- dS in e5m2 (one mantissa bit fewer: twice e4m3's relative rounding error):
  max-abs <= 2 x 2 x 1e-1, relative Frobenius <= 1e-1;
- dK and dV of a KV head shared by G query heads sum G independent per-head
  terms: their max-abs bound is sqrt(G) times the above (dQ's is not).
A CPU emulation of the two quantisations on these shapes gives max-abs errors
of 0.08-0.16 (e4m3 dS) and 0.14-0.37 (e5m2 dS), relative Frobenius 0.027 and
0.055."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from oracle import attention_forward, attention_probs
from sdpa_inputs import Workload
from tests.parity import TOL, check_out, f64, oracle_bwd, rel_fro, say, to_gpu

pytestmark = pytest.mark.gpu

FMAX = {torch.float8_e4m3fn: 448.0, torch.float8_e5m2: 57344.0}


def _oracle_ds_amax(w, ins, causal, lq=None, lk=None, align="top_left", o=None):
    """max |dS| over the whole problem from the oracle's weights (dS = P * (dP - D));
    D from the oracle's exact O unless ``o`` (float64, (b, h_q, s_q, d)) is given."""
    q, k, v, do = (f64(ins[n], ins.get("descale_" + n)) for n in ("q", "k", "v", "do"))
    p = attention_probs(q, k, w.scale, causal, seq_len_q=lq, seq_len_kv=lk, align=align)
    vv = np.repeat(v, w.h_q // w.h_kv, axis=1)
    if o is None:
        o = p @ vv
    dvec = (do * o).sum(-1, keepdims=True)
    ds = p * (do @ np.swapaxes(vv, -1, -2) - dvec)
    if lq is not None:  # rows past lq take no part (the kernel never forms them)
        for bi in range(w.b):
            ds[bi, :, int(lq[bi]):] = 0.0
    return float(np.abs(ds).max())


def _scale_for(amax, ds_dtype):
    """Delayed-scaling choice: the power of two that maps amax just inside the format."""
    return 2.0 ** math.floor(math.log2(FMAX[ds_dtype] / amax))


def _fp8_fwd(w, g, causal, lq=None, lk=None):
    fp8 = sdpa.Fp8Scales(g["descale_q"], g["descale_k"], g["descale_v"], g["scale_p"], g["descale_p"])
    o, lse = sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=causal, fp8=fp8, seq_len_q=lq,
                      seq_len_kv=lk)
    return o, lse


def _fp8_bwd(w, g, o, lse, causal, scale_ds, lq=None, lk=None, ds_dtype=torch.float8_e4m3fn, amax=None):
    dq, dk, dv = sdpa.bwd_fp8(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=causal,
                              descale_q=g["descale_q"], descale_k=g["descale_k"], descale_v=g["descale_v"],
                              descale_do=g["descale_do"], scale_ds=scale_ds, ds_dtype=ds_dtype, amax_ds=amax,
                              seq_len_q=lq, seq_len_kv=lk)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check(grads, refs, tol, rf_tol, tag="", group=1):
    """dK and dV of a KV head sum the contributions of its `group` query heads,
    whose quantisation errors (P and dS rounded per element) are independent:
    their bound is sqrt(group) times the per-head one; dQ keeps the plain bound."""
    for name, x, r in zip(("dq", "dk", "dv"), grads, refs):
        assert x.dtype == torch.bfloat16
        xa = f64(x.cpu())
        t = tol if name == "dq" else tol * math.sqrt(group)
        check_out(xa, r, t, grad_dtype="bf16", what=f"{tag}{name}: ")
        rf = rel_fro(xa, r)
        assert rf <= rf_tol, (name, rf)


def _run(w, causal=None, lens=None, seed=0, ds_dtype=torch.float8_e4m3fn):
    causal = w.causal if causal is None else causal
    say(f"[fp8 bwd] {w} causal={causal} lens={lens is not None} ds={ds_dtype}")
    ins = sdpa_inputs.make_inputs(w)
    assert ins["do"].dtype == torch.float8_e5m2
    g = to_gpu(ins)
    lq = lk = None
    if lens is not None:
        lq = sdpa_inputs.make_lengths(w.b, w.s_q, seed, min_len=lens)
        lk = sdpa_inputs.make_lengths(w.b, w.s_kv, seed + 1, min_len=lens)
    lqg = None if lq is None else lq.cuda()
    lkg = None if lk is None else lk.cuda()
    align = "bottom_right" if causal == "bottom_right" else "top_left"
    lqn = None if lq is None else lq.numpy()
    lkn = None if lk is None else lk.numpy()
    sds = _scale_for(_oracle_ds_amax(w, ins, bool(causal), lqn, lkn, align), ds_dtype)
    o, lse = _fp8_fwd(w, g, causal, lqg, lkg)
    grads = _fp8_bwd(w, g, o, lse, causal, sds, lqg, lkg, ds_dtype=ds_dtype)
    refs = oracle_bwd(w, ins, seq_len_q=lqn, seq_len_kv=lkn, align=align)
    widen = 2 if ds_dtype == torch.float8_e5m2 else 1
    _check(grads, refs, widen * 2 * TOL["fp8"], TOL["fp8"], group=w.h_q // w.h_kv)
    return ins, g, grads


def _fp8_workload(name, b, h_q, h_kv, s_q, s_kv, d, causal, layout, seed):
    return Workload(name, b, h_q, h_kv, s_q, s_kv, d, "fp8", "bf16", causal, 1 / math.sqrt(d), layout, seed,
                    backward=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_bwd_small(causal):
    _run(_fp8_workload("fp8_bwd", 2, 4, 4, 300, 300, 128, causal, "bshd", 31))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_bwd_e5m2_ds(causal):
    """dS quantised to e5m2, the format the recipe names for backward-pass tensors."""
    _run(_fp8_workload("fp8_bwd_e5m2ds", 2, 4, 2, 300, 300, 128, causal, "bshd", 33), ds_dtype=torch.float8_e5m2)


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
    (O rounded to bf16), so only the backward's own quantisation of P and dS
    remains."""
    w = _fp8_workload("fp8_bwd_d64", 2, 4, 2, 257, 257, 64, causal, "bshd", 64)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    q, k, v = (f64(ins[n], ins["descale_" + n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = attention_forward(q, k, v, w.scale, causal)
    o = sdpa_inputs.to_device_like(torch.from_numpy(o_ref).to(torch.bfloat16), "cuda")
    lse = torch.from_numpy(lse_ref).float().contiguous().cuda()
    sds = _scale_for(_oracle_ds_amax(w, ins, causal), torch.float8_e4m3fn)
    grads = _fp8_bwd(w, g, o, lse, causal, sds)
    _check(grads, oracle_bwd(w, ins), 2 * TOL["fp8"], TOL["fp8"], group=w.h_q // w.h_kv)


def test_fp8_bwd_amax_matches_oracle():
    """The reported max |dS| (before scaling and saturation) is the oracle's,
    computed with the same O the kernel gets (the bf16 O of the oracle's
    forward) and exact LSE: only fp32 rounding in S, dP and D remains. The
    report max-combines with what the buffer holds."""
    w = _fp8_workload("fp8_bwd_amax", 2, 4, 2, 190, 230, 128, True, "bhsd", 41)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    q, k, v = (f64(ins[n], ins["descale_" + n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = attention_forward(q, k, v, w.scale, True)
    o16 = torch.from_numpy(o_ref).to(torch.bfloat16)
    o = sdpa_inputs.to_device_like(o16, "cuda")
    lse = torch.from_numpy(lse_ref).float().contiguous().cuda()
    want = _oracle_ds_amax(w, ins, True, o=f64(o16))
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    _fp8_bwd(w, g, o, lse, True, _scale_for(want, torch.float8_e4m3fn), amax=amax)
    got = amax.item()
    say(f"    amax kernel={got:.6g} oracle={want:.6g}")
    assert abs(got - want) <= 1e-3 * want, (got, want)
    big = torch.full((1,), 1e6, dtype=torch.float32, device="cuda")  # larger than any |dS| here: kept
    _fp8_bwd(w, g, o, lse, True, 1.0, amax=big)
    assert big.item() == 1e6


def test_fp8_bwd_saturates_large_scale():
    """A scale_ds far too large saturates dS at the format's largest value
    instead of producing inf or NaN; the amax report still sees the true max."""
    w = _fp8_workload("fp8_bwd_sat", 1, 2, 2, 130, 130, 128, True, "bshd", 8)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = _fp8_fwd(w, g, True)
    for dt in (torch.float8_e4m3fn, torch.float8_e5m2):
        amax = torch.zeros(1, dtype=torch.float32, device="cuda")
        grads = _fp8_bwd(w, g, o, lse, True, 2.0 ** 40, ds_dtype=dt, amax=amax)
        for x in grads:
            assert torch.isfinite(x.float()).all()
        want = _oracle_ds_amax(w, ins, True)
        assert abs(amax.item() - want) <= 0.05 * want, (amax.item(), want)


def test_fp8_bwd_e4m3_gradient():
    """dO given in e4m3 instead of e5m2 (the all-E4M3 recipe)."""
    w = _fp8_workload("fp8_bwd_e4m3do", 1, 4, 4, 190, 190, 128, True, "bshd", 12)
    ins = sdpa_inputs.make_inputs(w)
    do32 = f64(ins["do"], ins["descale_do"])
    ins["do"], ins["descale_do"] = sdpa_inputs.quantize_fp8(torch.from_numpy(do32).float(), "e4m3")
    g = to_gpu(ins)
    sds = _scale_for(_oracle_ds_amax(w, ins, True), torch.float8_e4m3fn)
    o, lse = _fp8_fwd(w, g, True)
    grads = _fp8_bwd(w, g, o, lse, True, sds)
    _check(grads, oracle_bwd(w, ins), 2 * TOL["fp8"], TOL["fp8"])


def test_fp8_bwd_matches_scaled_codes():
    """Factors fold in exactly: doubling dO's descale while halving scale_ds
    (both powers of two, exact in fp32) leaves every quantised dS code as it
    was and doubles all three gradients bit for bit, since each is linear in dO
    and the factors only enter fp32 scalars."""
    w = _fp8_workload("fp8_bwd_fold", 1, 2, 2, 130, 130, 128, True, "bshd", 3)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = _fp8_fwd(w, g, True)
    sds = _scale_for(_oracle_ds_amax(w, ins, True), torch.float8_e4m3fn)
    base = _fp8_bwd(w, g, o, lse, True, sds)
    g2 = dict(g, descale_do=g["descale_do"] * 2)
    twice = _fp8_bwd(w, g2, o, lse, True, sds / 2)
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
    sdpa.bwd_fp8(q, k, k, o, do, lse, scale=w.scale, descale_q=1.0, descale_k=1.0, descale_v=1.0, scale_ds=1.0,
                 descale_do=1.0, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert dk.abs().max().item() == 0 and dv.abs().max().item() == 0


def test_fp8_bwd_full_size_sampled():
    """b2 h16 s8192 d128 causal (the hd128 training shape) in fp8: two KV heads'
    gradients. scale_ds comes the recipe's way: a first backward with scale 1
    reports max |dS| (no oracle can form all of dS at this size), and the
    second backward runs with the power of two that maps it inside e4m3."""
    w = sdpa_inputs.fp8_hd128()
    say(f"[fp8 bwd sampled] {w}")
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = _fp8_fwd(w, g, True)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    _fp8_bwd(w, g, o, lse, True, 1.0, amax=amax)
    sds = _scale_for(amax.item(), torch.float8_e4m3fn)
    say(f"    amax={amax.item():.4g} scale_ds={sds:g}")
    grads = _fp8_bwd(w, g, o, lse, True, sds)
    groups = [(0, 3), (w.b - 1, w.h_kv - 1)]
    refs = oracle_bwd(w, ins, kv_heads=groups)
    _check(grads, refs, 2 * TOL["fp8"], TOL["fp8"], tag=f"groups={groups} ")
