"""GPU parity of dropout (Philox4x32-10 mask regenerated in the backward)
against the float64 oracle, which builds the same mask from the same rule.

The value checks compare O and the gradients within the tolerances; the
keep masks themselves are integer work and are compared bit for bit: each
kernel's mask (forward, dK/dV, dQ) is read back through inputs that make
one output element's zero pattern or sign depend on exactly one mask bit."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from oracle import attention_backward, attention_forward, dropout_mask
from sdpa_inputs import Workload
from tests.parity import LSE_REL, TOL, check_out, f64, say, to_gpu

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
    check_out(f64(o.cpu()), o_ref, TOL[w.out_dtype], what="O: ")


def _check_lse(lg, lr):
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr))
    fin = np.isfinite(lr)
    err = np.abs(lg[fin] - lr[fin]) / np.maximum(1.0, np.abs(lr[fin]))
    assert err.max() <= LSE_REL


def _check_grads(w, grads, refs):
    for name, x, r in zip(("dq", "dk", "dv"), grads, refs):
        check_out(f64(x.cpu()), r, 2 * TOL[w.out_dtype], grad_dtype=w.out_dtype, what=f"{name}: ")


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


# ---------------------------------------------------------------------------
# Bit-exact keep masks. The keep decision is integer work (a random byte
# against k8), so each kernel's mask is read back exactly through an input
# that makes one output element depend on one mask bit, and compared bit for
# bit with the oracle's dropout_mask (which builds it from the published
# Philox4x32-10 definition). Rows and keys reach the sizes of the
# b2 h16 s8192 workload, so the row and key counters pass 2^11.
# ---------------------------------------------------------------------------

_HEADS = [(0, 0), (1, 15), (1, 6)]  # (b, h) slots checked: slot b * 16 + h


def _identity_rows(w, n, device="cuda"):
    """(b, h, n, d) tensor in w's layout whose row i is the unit vector e_i (n <= d)."""
    x = sdpa_inputs.empty_logical(w.b, w.h_q, n, w.d, w.layout, w.dtype)
    x.zero_()
    idx = torch.arange(n)
    x[:, :, idx, idx] = 1
    return sdpa_inputs.to_device_like(x, device)


@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f16")])
def test_forward_keep_mask_bit_exact(d, dtype, mask):
    """s_kv = d and V = I: O_ij = P_ij Z_ij, so O_ij != 0 exactly where key j
    of row i is kept (every visible weight is > 0 for N(0,1) scores)."""
    w = Workload("drop_fwd_mask", 2, 16, 16, 8192, d, d, dtype, dtype, mask != "none", 1 / math.sqrt(d), "bshd",
                 1300 + d)
    drop = _drop(0.1, 0xC0FFEE123456789, 77)
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    g["v"] = _identity_rows(w, d)
    say(f"[dropout fwd mask] {w} mask={mask}")
    o, _, _ = _run(w, g, mask, drop, False)
    oc = o.cpu()
    rows = np.arange(w.s_q)
    for bi, hq in _HEADS:
        z = dropout_mask(bi * w.h_q + hq, rows, d, drop["dropout_p"], drop["dropout_seed"], drop["dropout_offset"])
        visible = np.ones((w.s_q, d), dtype=bool) if mask == "none" else (np.arange(d)[None, :] <= rows[:, None])
        got = (oc[bi, hq].float().numpy() != 0)
        assert np.array_equal(got, (z > 0) & visible), (bi, hq, int((got != ((z > 0) & visible)).sum()))
        say(f"    slot ({bi},{hq}): {int(got.sum())} kept of {int(visible.sum())} visible, mask identical")


@pytest.mark.parametrize("mask", ["none", "bottom_right"])
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f16")])
def test_dkdv_keep_mask_bit_exact(d, dtype, mask):
    """s_q = d and dO = I: dV_j = sum_i P_ij Z_ij dO_i gives dV[j, i] = P_ij Z_ij,
    so the dK/dV kernel's regenerated mask is dV^T's nonzero pattern."""
    w = Workload("drop_dkdv_mask", 2, 16, 16, d, 8192, d, dtype, dtype, mask != "none", 1 / math.sqrt(d), "bshd",
                 1400 + d, backward=True)
    drop = _drop(0.1, 0x1234ABCD5678, 5)
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    g["do"] = _identity_rows(w, d)
    say(f"[dropout dK/dV mask] {w} mask={mask}")
    _, _, (dq, dk, dv) = _run(w, g, mask, drop, True)
    dvc = dv.cpu()
    rows = np.arange(w.s_q)
    keys = np.arange(w.s_kv)
    visible = np.ones((w.s_q, w.s_kv), dtype=bool) if mask == "none" else \
        keys[None, :] <= rows[:, None] + (w.s_kv - w.s_q)
    for bi, hq in _HEADS:
        z = dropout_mask(bi * w.h_q + hq, rows, w.s_kv, drop["dropout_p"], drop["dropout_seed"],
                         drop["dropout_offset"])
        got = (dvc[bi, hq].float().numpy().T != 0)  # [i, j]
        assert np.array_equal(got, (z > 0) & visible), (bi, hq, int((got != ((z > 0) & visible)).sum()))
        say(f"    slot ({bi},{hq}): {int(got.sum())} kept of {int(visible.sum())} visible, mask identical")


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f16")])
def test_dq_keep_mask_bit_exact(d, dtype):
    """Q = 0 (P = 1/s_kv), K = I (s_kv = d), dO_i = e_0 and V_j0 = 1, so
    dP_ij = 1, D_i = mean_j Z_ij and dQ_ij = scale * dS_ij =
    (scale / s_kv) (Z_ij - mean_j Z_ij): positive exactly where kept (p = 0.25
    makes a row with every key kept, where all would be 0, practically
    impossible). The sign of dQ is the dQ kernel's mask."""
    w = Workload("drop_dq_mask", 2, 16, 16, 8192, d, d, dtype, dtype, False, 1 / math.sqrt(d), "bshd",
                 1500 + d, backward=True)
    drop = _drop(0.25, 0xFEEDFACE0042, 9)
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    ins["q"] = torch.zeros_like(ins["q"])
    ins["v"][:, :, :, 0] = 1
    ins["do"].zero_()
    ins["do"][:, :, :, 0] = 1
    g = to_gpu(ins)
    g["k"] = _identity_rows(w, d)
    say(f"[dropout dQ mask] {w}")
    _, _, (dq, dk, dv) = _run(w, g, "none", drop, True)
    dqc = dq.cpu().float().numpy()
    rows = np.arange(w.s_q)
    for bi, hq in _HEADS:
        z = dropout_mask(bi * w.h_q + hq, rows, d, drop["dropout_p"], drop["dropout_seed"], drop["dropout_offset"])
        assert (z > 0).sum(axis=1).max() < d  # no row with every key kept
        got = dqc[bi, hq]
        assert (got != 0).all()
        assert np.array_equal(got > 0, z > 0), (bi, hq, int(((got > 0) != (z > 0)).sum()))
        say(f"    slot ({bi},{hq}): {int((got > 0).sum())} kept of {got.size}, mask identical")
