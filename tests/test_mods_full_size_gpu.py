"""Full-size parity of the score modifiers at the hd128 causal training shape
(b2 h16 s8192 d128 bf16 BSHD, the shape whose training step with ALiBi and
with dropout 0.1 the benchmark times). The kernels run at full size; the
oracle checks sampled rows of sampled heads in the forward and whole sampled
KV groups in the backward. ALiBi distances reach 8191 and the Philox row and
key counters pass 2^11 at this size."""
import numpy as np
import pytest
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from oracle import attention_backward, attention_forward
from tests.parity import LSE_REL, TOL, check_out, f64, say, to_gpu

pytestmark = pytest.mark.gpu


def _rows(s, rng, n=40):
    return np.array(sorted(set([0, 1, 127, 128, 255, 256, s // 2, s - 2, s - 1]
                               + [int(x) for x in rng.integers(0, s, n)])))


def _full_size(mods_gpu: dict, mods_oracle: dict, n_groups: int, seed: int):
    w = sdpa_inputs.hd128(8192)
    say(f"[mods full size] {w} mods={sorted(mods_gpu)}")
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    g = to_gpu(ins)
    o, lse = sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=True, **mods_gpu)
    dq, dk, dv = sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=True, **mods_gpu)
    torch.cuda.synchronize()
    q, k, v, do = (f64(ins[n]) for n in ("q", "k", "v", "do"))
    rng = np.random.default_rng(seed)

    heads = [(0, 0), (w.b - 1, w.h_q - 1), (int(rng.integers(w.b)), int(rng.integers(w.h_q)))]
    rows = _rows(w.s_q, rng)
    o_ref, lse_ref = attention_forward(q, k, v, w.scale, True, heads=heads, rows=rows, **mods_oracle)
    check_out(f64(o.cpu())[:, :, rows], o_ref, TOL["bf16"], what=f"O heads={heads}: ")
    lg = lse.cpu().numpy()[:, :, rows]
    m = ~np.isnan(lse_ref)
    err = np.abs(lg[m] - lse_ref[m]) / np.maximum(1.0, np.abs(lse_ref[m]))
    say(f"    LSE rel err {err.max():.3e}")
    assert err.max() <= LSE_REL

    groups = [(w.b - 1, w.h_kv - 1)] + [(int(rng.integers(w.b)), int(rng.integers(w.h_kv)))
                                        for _ in range(n_groups - 1)]
    refs = attention_backward(q, k, v, do, w.scale, True, kv_heads=groups, **mods_oracle)
    for name, x, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        check_out(f64(x.cpu()), r, 2 * TOL["bf16"], grad_dtype="bf16", what=f"{name} groups={groups}: ")


def test_alibi_full_size_sampled():
    slopes = sdpa.alibi_slopes(16, device="cpu")
    _full_size(dict(alibi_slopes=slopes.cuda()), dict(alibi_slopes=slopes.double().numpy()), 2, 1)


def test_dropout_full_size_sampled():
    drop = dict(dropout_p=float(np.float32(0.1)), dropout_seed=0x5EED5EED, dropout_offset=12)
    _full_size(drop, drop, 1, 2)


def test_bias_and_alibi_full_size_sampled():
    """A (1, 1, s, s) bf16 bias broadcast over batch and heads, plus ALiBi:
    the general modifier kernels (bias loads)."""
    bias = sdpa_inputs.make_bias((1, 1, 8192, 8192), 77, "bf16")
    slopes = sdpa.alibi_slopes(16, device="cpu")
    _full_size(dict(bias=bias.cuda(), alibi_slopes=slopes.cuda()),
               dict(bias=bias.float().numpy(), alibi_slopes=slopes.double().numpy()), 1, 3)
