"""GPU parity of the fp8 (e4m3) forward against the float64 oracle.

The oracle receives the dequantised inputs (e4m3 code x per-tensor descale)
and computes the exact softmax; the kernel quantises P to e4m3 for the second
matmul, which is what the fp8 tolerance absorbs. Checks: max-abs error beyond
bf16 output rounding <= 1e-1, relative Frobenius error <= 1e-1 (a max-abs bound
alone would pass an all-zero output at long sequence lengths, where |O| is
small), and LSE within 1e-3 relative (it does not involve the quantised P)."""
import math

import numpy as np
import torch
import pytest

import sdpa_inputs
from sdpa_inputs import Workload
from tests.parity import TOL, check_lse, check_out, f64, gpu_fwd, oracle_fwd, rel_fro, say, to_gpu

pytestmark = pytest.mark.gpu


def _check(w, o, lse, o_ref, lse_ref, rows=None):
    og = f64(o.cpu())
    lg = lse.cpu().numpy()
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    check_out(og, o_ref, TOL["fp8"], what=f"fp8 O (max|O|={np.nanmax(np.abs(o_ref)):.3f}): ")
    rf = rel_fro(og, o_ref)
    assert rf <= TOL["fp8"], rf
    check_lse(lg, lse_ref)
    return rf


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_small(d, causal):
    w = Workload("fp8_small", 2, 4, 4, 300, 300, d, "fp8", "bf16", causal, 1 / math.sqrt(d), "bshd", 17 + d)
    say(f"[fp8] {w}")
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = gpu_fwd(w, g)
    o_ref, lse_ref = oracle_fwd(w, ins)
    rf = _check(w, o, lse, o_ref, lse_ref)
    # e4m3 P carries 3 mantissa bits: the relative error is a few percent, not zero
    assert rf > 1e-4


def test_fp8_gqa_ragged():
    w = Workload("fp8_gqa", 1, 8, 2, 161, 230, 256, "fp8", "bf16", False, 1 / 16, "bhsd", 3)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = gpu_fwd(w, g)
    o_ref, lse_ref = oracle_fwd(w, ins)
    _check(w, o, lse, o_ref, lse_ref)


def test_fp8_hd256_full_size_sampled():
    """b4 h8 s8192 d256 non-causal (the cuDNN 9 blog's fp8 figure shape): sampled rows."""
    w = sdpa_inputs.fp8()
    say(f"[fp8 sampled] {w}")
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    o, lse = gpu_fwd(w, g)
    rng = np.random.default_rng(0)
    heads = [(0, 0), (w.b - 1, w.h_q - 1), (2, 5)]
    rows = sorted(set([0, 1, 63, 64, 4095, w.s_q - 1] + [int(x) for x in rng.integers(0, w.s_q, 40)]))
    o_ref, lse_ref = oracle_fwd(w, ins, heads=heads, rows=np.array(rows))
    _check(w, o, lse, o_ref, lse_ref, rows=rows)


@pytest.mark.parametrize("beta", [14.7, -7.0])
def test_fp8_late_dominant_key(beta):
    """One key of a row, in a later 64-key tile, scores 0.4-2.7 (log2 units) above (beta > 0)
    or below (beta < 0) the first tile's max; V is +4 on key 0 and -4 on that key. With the
    exact running max the larger of the two weights is exactly scale_p; a max that trails the
    row max (moved only past a threshold) left it to e4m3 rounding and O off by up to 0.14.
    Scores are scale * alpha_i * b_j on one coordinate: key 0 gives 0, key 150 gives
    beta * scale * alpha_i, every other key at most -8.8 nats."""
    b, h, s, d = 1, 1, 256, 128
    w = Workload("fp8_late_max", b, h, h, s, s, d, "fp8", "bf16", False, 1 / math.sqrt(d), "bhsd", 0)
    q = torch.zeros(b, h, s, d)
    k = torch.zeros(b, h, s, d)
    alpha = 0.5 + torch.arange(s, dtype=torch.float32) / s
    q[0, 0, :, 0] = alpha
    k[0, 0, :, 0] = -200.0
    k[0, 0, 0, 0] = 0.0
    k[0, 0, 150, 0] = beta
    v = torch.randn(b, h, s, d, generator=torch.Generator().manual_seed(5)) * 0.1
    v[0, 0, 0, :] = 4.0
    v[0, 0, 150, :] = -4.0
    ins = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        ins[name], ins["descale_" + name] = sdpa_inputs.quantize_fp8(x)
    ins["scale_p"] = sdpa_inputs.FP8_MAX
    ins["descale_p"] = 1.0 / sdpa_inputs.FP8_MAX
    o, lse = gpu_fwd(w, to_gpu(ins))
    o_ref, lse_ref = oracle_fwd(w, ins)
    _check(w, o, lse, o_ref, lse_ref)
