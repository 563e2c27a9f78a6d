"""GPU parity of the backward kernels (dQ, dK, dV) against the float64 oracle.

The kernel's backward consumes the kernel's own forward output O and LSE; the
oracle recomputes everything from Q, K, V, dO in float64. Tolerance: twice the
forward's max-abs bound for the dtype."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from sdpa_inputs import Workload
from tests.parity import TOL, check_out, f64, gpu_fwd, oracle_bwd, say, to_gpu

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(w, g):
    o, lse = gpu_fwd(w, g)
    dq, dk, dv = sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _check(w, grads, refs, tag=""):
    tol = 2 * TOL[w.out_dtype]
    for name, x, r in zip(("dq", "dk", "dv"), grads, refs):
        check_out(f64(x.cpu()), r, tol, grad_dtype=w.out_dtype, what=f"{tag}{name}: ")


def _run_full(w: Workload):
    say(f"[bwd] {w}")
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    _, _, dq, dk, dv = gpu_fwd_bwd(w, g)
    _check(w, (dq, dk, dv), oracle_bwd(w, ins))
    return ins, g, (dq, dk, dv)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_ragged_mha(dtype, d, causal):
    w = Workload("bwd", 2, 3, 3, 333, 333, d, dtype, dtype, causal, 1 / math.sqrt(d), "bshd", 21 + d)
    _run_full(w)


@pytest.mark.parametrize("h_kv", [4, 2, 1])
@pytest.mark.parametrize("causal", [False, True])
def test_small_gqa_split(h_kv, causal):
    """Small GQA/MQA problems take the split-group path (fp32 partials + reduce)."""
    w = Workload("bwd_gqa", 1, 8, h_kv, 200, 200, 128, "bf16", "bf16", causal, 1 / math.sqrt(128), "bhsd", h_kv)
    _run_full(w)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,skv", [(100, 260), (260, 100), (1, 70)])
def test_unequal_lengths(causal, sq, skv):
    w = Workload("bwd_uneq", 1, 2, 1, sq, skv, 128, "bf16", "bf16", causal, 0.09, "bshd", 4)
    _run_full(w)


def _sampled(w: Workload, n_groups=1, seed=0):
    say(f"[bwd sampled] {w}")
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    _, _, dq, dk, dv = gpu_fwd_bwd(w, g)
    rng = np.random.default_rng(seed)
    groups = [(w.b - 1, w.h_kv - 1)] + [(int(rng.integers(w.b)), int(rng.integers(w.h_kv)))
                                       for _ in range(n_groups - 1)]
    refs = oracle_bwd(w, ins, kv_heads=groups)
    _check(w, (dq, dk, dv), refs, tag=f"groups={groups} ")


@pytest.mark.parametrize("s", sdpa_inputs.HD128_SEQS)
def test_hd128_causal_full_size_sampled(s):
    _sampled(sdpa_inputs.hd128(s), n_groups=3, seed=s)


@pytest.mark.parametrize("h_kv", [32, 8, 1])
def test_gqa_full_size_sampled(h_kv):
    _sampled(sdpa_inputs.gqa(h_kv), n_groups=2 if h_kv > 1 else 1, seed=h_kv)


def test_invariants():
    """Rows of dS sum to zero, so sum_j dK_j = 0; constant V gives dQ = dK = 0;
    causal row 0 has dQ_0 = 0 (it sees one key)."""
    w = Workload("inv", 1, 4, 2, 256, 256, 128, "bf16", "bf16", True, 1 / math.sqrt(128), "bshd", 8)
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    _, _, dq, dk, dv = gpu_fwd_bwd(w, g)
    assert dk.float().sum(dim=2).abs().max().item() < 0.05
    assert dq[:, :, 0].float().abs().max().item() < 1e-3
    ins["v"] = torch.full_like(ins["v"], 0.75)
    g = to_gpu(ins)
    _, _, dq, dk, dv = gpu_fwd_bwd(w, g)
    assert dq.float().abs().max().item() < 1e-3 and dk.float().abs().max().item() < 1e-3


def test_deterministic():
    w = sdpa_inputs.gqa(1)
    w.s_q = w.s_kv = 1024
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    a = gpu_fwd_bwd(w, g)
    b = gpu_fwd_bwd(w, g)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_no_query_rows_gives_zero_dkdv():
    w = Workload("e", 1, 4, 2, 0, 64, 128, "bf16", "bf16", True, 0.1, "bshd", 1)
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    o = torch.empty_like(g["q"])
    lse = torch.empty((1, 4, 0), device="cuda")
    dk = torch.full_like(g["k"], 3.0)
    dv = torch.full_like(g["v"], 3.0)
    sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=True, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert dk.abs().max().item() == 0 and dv.abs().max().item() == 0


def test_workspace_too_small_is_reported():
    w = Workload("ws", 1, 2, 2, 64, 64, 128, "bf16", "bf16", True, 0.1, "bshd", 1)
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    o, lse = gpu_fwd(w, g)
    with pytest.raises(sdpa.SdpaError, match="WORKSPACE_TOO_SMALL"):
        sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=True,
                 workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
