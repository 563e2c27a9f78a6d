"""GPU parity of the forward's running-max handling against the float64 oracle.

Without score modifiers the kernel takes each tile's weights against the
running max as it stands (started from the row's score against key 0) and
moves the max only when a tile's weights grow past 2^8; a weight that
overflows fp32 makes the workgroup redo its rows on the exact path. These
inputs drive both: scores that climb steadily along the key index (the max
moves many times, by about 24 log2 units per 128-key tile), and rows whose key 0
scores ~0 while every other key scores ~147 log2 units (exp2 overflows fp32).
Q and K are built from a seeded random unit direction so that the scores are
exact multiples of its squared norm; V is the seeded N(0, 1) draw."""
import math

import pytest
import torch

import sdpa_inputs
from sdpa_inputs import Workload
from tests.parity import TOL, check_lse, check_out, f64, gpu_fwd, oracle_fwd, say, to_gpu

pytestmark = pytest.mark.gpu

_DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _structured(w: Workload, key_gain) -> dict:
    """q rows = 3 u, k rows = key_gain(j) u, for one seeded direction u with entries +-1 (so
    every product is exact in the io dtype); returns inputs in the layout of w."""
    ins = sdpa_inputs.make_inputs(w, with_grad=False)
    gen = torch.Generator().manual_seed(w.seed + 1000)
    u = torch.where(torch.rand(w.d, generator=gen) < 0.5, -1.0, 1.0)
    gains = torch.tensor([key_gain(j) for j in range(w.s_kv)], dtype=torch.float32)
    # Physical storage is BSHD or BHSD; write through the logical views.
    ins["q"].copy_((3.0 * u).expand_as(ins["q"]).to(ins["q"].dtype))
    ins["k"].copy_((gains[:, None] * u[None, :]).expand_as(ins["k"]).to(ins["k"].dtype))
    return ins


def _check(w: Workload, ins: dict):
    say(f"[fwd-max] {w}")
    g = to_gpu(ins)
    o, lse = gpu_fwd(w, g)
    o_ref, lse_ref = oracle_fwd(w, ins)
    got = f64(o.cpu())
    check_out(got, o_ref, TOL[w.out_dtype], what="O: ")
    check_lse(lse.cpu().numpy(), lse_ref)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 128), ("bf16", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_climb_along_keys(dtype, d, causal):
    """The row max grows tile after tile (the key gain rises by 1/16 every 16 keys: about 24
    log2 units per 128-key tile at d = 128), so the weights of most tiles outgrow the running
    max."""
    # 1100 keys: past 1024, the d = 128 forward runs its 8-wave, 128-key tile kernel.
    w = Workload("climb", 1, 2, 2, 1100, 1100, d, dtype, dtype, causal, 1 / math.sqrt(d), "bshd", 31)
    _check(w, _structured(w, lambda j: (j // 16) / 16.0 - 1.0))


@pytest.mark.parametrize("dtype,s,d", [("bf16", 300, 128), ("f16", 300, 128), ("bf16", 1030, 128),
                                       ("f16", 300, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_weight_overflow_redoes_rows(dtype, s, d, causal):
    """Key 0 scores 0; every other key scores 3 c d / sqrt(d) with c = 3 at d = 128 (101.8,
    146.9 in log2 units) and c = 4.5 at d = 64 (108, 155.8 in log2 units): past fp32's exp2
    range when taken against key 0's score. (At d = 64 the second key group of the split
    forward starts from key 64's score and overflows nothing; the first group's overflow
    sends the whole workgroup back.)"""
    w = Workload("ovf", 2, 2, 1, s, s, d, dtype, dtype, causal, 1 / math.sqrt(d), "bhsd", 32)
    c = 3.0 if d == 128 else 4.5
    _check(w, _structured(w, lambda j: 0.0 if j == 0 else c))


def test_overflow_in_some_heads_only():
    """One head overflows and is redone, the other takes the fast path; both must agree with
    the oracle (the redo is per workgroup)."""
    w = Workload("ovf2", 1, 2, 2, 520, 520, 128, "bf16", "bf16", True, 1 / math.sqrt(128), "bshd", 33)
    ins = _structured(w, lambda j: 0.0 if j == 0 else 3.0)
    rnd = sdpa_inputs.make_inputs(w, with_grad=False)
    ins["q"][:, 1].copy_(rnd["q"][:, 1])
    ins["k"][:, 1].copy_(rnd["k"][:, 1])
    _check(w, ins)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,skv", [(1, 300), (77, 1000), (300, 257), (130, 4100)])
def test_key_split_shapes(sq, skv, causal):
    """d = 64 shapes that take the two-group key split (few row blocks, >= 256 keys): a
    single query row, key counts that end mid-tile and mid-group, s_q != s_kv (top-left
    causal: rows see keys 0..i, so the second group sees nothing for the first rows)."""
    w = Workload("ksplit", 2, 3, 1, sq, skv, 64, "f16", "f16", causal, 0.125, "bshd", 34 + sq)
    _check(w, sdpa_inputs.make_inputs(w, with_grad=False))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_key_split_group_without_visible_keys(dtype):
    """Causal d = 64 key split: rows 0..63 see none of the second group's keys, whose first key
    (key 64) scores 155.8 log2 units above every key those rows see. That group's starting max
    is then a masked key's score, and its empty partial must not move the merged max (it would
    scale the first group's weights to zero)."""
    w = Workload("ksplit_empty", 1, 2, 2, 300, 300, 64, dtype, dtype, True, 0.125, "bshd", 35)
    _check(w, _structured(w, lambda j: 4.5 if 64 <= j < 128 else 0.0))
