"""GPU parity of the forward kernels against the float64 oracle (MI355X).

Small cases run the oracle on every output; the full-size workloads run the
kernel at full size and check sampled rows of sampled heads, which the oracle
computes one by one. Inputs come from sdpa_inputs (seeded, same bits on both
sides)."""
import math

import numpy as np
import pytest
import torch

import sdpa_inputs
from sdpa_inputs import Workload
from tests.parity import TOL, check_lse, check_out, f64, gpu_fwd, oracle_fwd, rel_fro, say, to_gpu

pytestmark = pytest.mark.gpu


def _run_full(w: Workload, check_lse_too=True):
    say(f"[fwd] {w}")
    ins = sdpa_inputs.make_inputs(w, with_grad=False)
    g = to_gpu(ins)
    o, lse = gpu_fwd(w, g)
    o_ref, lse_ref = oracle_fwd(w, ins)
    check_out(f64(o.cpu()), o_ref, TOL[w.out_dtype], what="O: ")
    if check_lse_too:
        check_lse(lse.cpu().numpy(), lse_ref)
    return o, lse, ins


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_fp32(causal):
    _run_full(sdpa_inputs.tiny(causal))


def test_gpt2_fp16_full():
    """b4 h12 s1024 d64 fp16 BSHD causal, scale 1/8 (the GPT-2-like page example), every output."""
    _run_full(sdpa_inputs.gpt2())


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_small_ragged(dtype, d, causal, layout):
    """Several tiles plus a ragged tail in both s_q and s_kv."""
    w = Workload("ragged", 2, 4, 2, 333, 333, d, dtype, dtype, causal, 1 / math.sqrt(d), layout, 7 + d)
    _run_full(w)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,skv", [(100, 260), (260, 100), (1, 77), (129, 1)])
def test_unequal_lengths(causal, sq, skv):
    """s_q != s_kv, top-left causal alignment."""
    w = Workload("uneq", 1, 2, 1, sq, skv, 128, "bf16", "bf16", causal, 0.09, "bshd", 3)
    _run_full(w)


@pytest.mark.parametrize("h_kv", [8, 2, 1])
def test_gqa_small(h_kv):
    w = Workload("gqa", 1, 8, h_kv, 300, 300, 128, "bf16", "bf16", True, 1 / math.sqrt(128), "bshd", h_kv)
    _run_full(w)


def test_fp32_d128_and_gqa():
    w = Workload("f32", 1, 4, 2, 150, 150, 128, "f32", "f32", True, 0.1, "bhsd", 11)
    _run_full(w)


def _sampled(w: Workload, n_heads=3, n_rows=48, seed=0):
    """Full-size launch; oracle on sampled heads and rows (first, last, tile edges, random)."""
    say(f"[fwd sampled] {w}")
    ins = sdpa_inputs.make_inputs(w, with_grad=False)
    g = to_gpu(ins)
    o, lse = gpu_fwd(w, g)
    rng = np.random.default_rng(seed)
    heads = [(0, 0), (w.b - 1, w.h_q - 1)] + [(int(rng.integers(w.b)), int(rng.integers(w.h_q)))
                                              for _ in range(n_heads - 2)]
    rows = sorted(set([0, 1, 63, 64, 127, 128, w.s_q // 2, w.s_q - 2, w.s_q - 1]
                      + [int(x) for x in rng.integers(0, w.s_q, n_rows)]))
    o_ref, lse_ref = oracle_fwd(w, ins, heads=heads, rows=np.array(rows))
    o_gpu = f64(o.cpu())[:, :, rows]
    tol = TOL["fp8"] if w.dtype == "fp8" else TOL[w.out_dtype]
    check_out(o_gpu, o_ref, tol, what=f"O heads={heads}: ")
    check_lse(lse.cpu().numpy()[:, :, rows], lse_ref)
    return o, lse, ins, rel_fro(o_gpu, o_ref)


@pytest.mark.parametrize("s", sdpa_inputs.HD128_SEQS)
def test_hd128_causal_full_size_sampled(s):
    _sampled(sdpa_inputs.hd128(s))


@pytest.mark.parametrize("h_kv", [32, 8, 1])
def test_gqa_full_size_sampled(h_kv):
    _sampled(sdpa_inputs.gqa(h_kv))


def test_causal_row0_is_v0_and_last_row_matches_full():
    """Invariants on kernel output: causal row 0 returns V[0] exactly; the last row is the same
    with and without the mask (JAX attention codelab, step 7)."""
    w = Workload("inv", 2, 4, 4, 256, 256, 128, "bf16", "bf16", True, 1 / math.sqrt(128), "bshd", 5)
    ins = sdpa_inputs.make_inputs(w, with_grad=False)
    g = to_gpu(ins)
    oc, lc = gpu_fwd(w, g)
    w.causal = False
    on, ln = gpu_fwd(w, g)
    assert torch.equal(oc[:, :, 0].cpu(), ins["v"][:, :, 0])
    assert (oc[:, :, -1].float() - on[:, :, -1].float()).abs().max().item() <= 2e-2
    assert (oc[:, :, 0].float() - on[:, :, 0].float()).abs().max().item() > 0.1


def test_q_zero_gives_column_mean():
    w = Workload("qz", 1, 2, 2, 200, 200, 128, "bf16", "bf16", False, 0.1, "bshd", 6)
    ins = sdpa_inputs.make_inputs(w, with_grad=False)
    ins["q"] = torch.zeros_like(ins["q"])
    g = to_gpu(ins)
    o, lse = gpu_fwd(w, g)
    mean = ins["v"].double().mean(dim=2, keepdim=True)
    assert (o.cpu().double() - mean).abs().max().item() <= 2e-2
    assert (lse.cpu().double() - math.log(200)).abs().max().item() <= 1e-3 * math.log(200)


def test_bshd_equals_bhsd_and_inference_mode():
    w = Workload("lay", 2, 4, 2, 300, 300, 128, "bf16", "bf16", True, 0.1, "bshd", 9)
    ins = sdpa_inputs.make_inputs(w, with_grad=False)
    g = to_gpu(ins)
    o1, l1 = gpu_fwd(w, g)
    g2 = {k: (v.contiguous() if isinstance(v, torch.Tensor) else v) for k, v in g.items()}
    assert g2["q"].stride() != g["q"].stride()
    o2, l2 = gpu_fwd(w, g2)
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(l1.cpu(), l2.cpu())
    o3, l3 = gpu_fwd(w, g, return_lse=False)
    assert l3 is None and torch.equal(o1.cpu(), o3.cpu())


def test_deterministic():
    w = sdpa_inputs.hd128(2048)
    ins = sdpa_inputs.make_inputs(w, with_grad=False)
    g = to_gpu(ins)
    o1, l1 = gpu_fwd(w, g)
    o2, l2 = gpu_fwd(w, g)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_problem():
    w = Workload("empty", 0, 2, 2, 64, 64, 128, "bf16", "bf16", True, 0.1, "bshd", 1)
    ins = sdpa_inputs.make_inputs(w, with_grad=False)
    g = to_gpu(ins)
    o, lse = gpu_fwd(w, g)
    assert o.numel() == 0
