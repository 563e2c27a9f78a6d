"""GPU test of sdpa_fwd_noalloc, the forward entry point that allocates
nothing: called through the C ABI, its output must equal sdpa_fwd_ex's with a
caller workspace on the same inputs (the same kernels and split plan, so
bitwise), on two calls in a row, the second with a smaller problem (the static
scratch keeps the first call's partials), and it must reject a shape whose
split-KV partials exceed its scratch before launching anything."""
import ctypes
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from oracle import attention_forward
from sdpa_inputs import Workload
from tests.parity import TOL, check_out, f64, say, to_gpu

pytestmark = pytest.mark.gpu

S = ctypes.c_int64 * 4


def _args(g, o, lse, w):
    return (ctypes.c_void_p(g["q"].data_ptr()), ctypes.c_void_p(g["k"].data_ptr()), ctypes.c_void_p(g["v"].data_ptr()),
            ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()), w.b, w.h_q, w.h_kv, w.s_q, w.s_kv, w.d,
            S(*g["q"].stride()), S(*g["k"].stride()), S(*g["v"].stride()), S(*o.stride()), float(w.scale),
            sdpa.SDPA_MASK_CAUSAL if w.causal else sdpa.SDPA_MASK_NONE, None, None, None, sdpa.SDPA_BF16,
            sdpa.SDPA_BF16, None)


def _both(w):
    lib = sdpa.load_library()
    ins = sdpa_inputs.make_inputs(w)
    g = to_gpu(ins)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n_ws = sdpa.fwd_workspace_size(w.b, w.h_q, w.h_kv, w.s_q, w.s_kv, w.d, torch.bfloat16)
    assert n_ws > 0, "the shape must take the split-KV path with a workspace"
    ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    o_ref = torch.empty_like(g["q"])
    l_ref = torch.empty((w.b, w.h_q, w.s_q), dtype=torch.float32, device="cuda")
    st = lib.sdpa_fwd_ex(*_args(g, o_ref, l_ref, w), ctypes.c_void_p(ws.data_ptr()), n_ws, stream)
    assert st == 0, lib.sdpa_last_error().decode()
    o = torch.full_like(g["q"], float("nan"))
    lse = torch.full((w.b, w.h_q, w.s_q), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.sdpa_fwd_noalloc(*_args(g, o, lse, w), stream)
    assert st == 0, lib.sdpa_last_error().decode()
    torch.cuda.synchronize()
    say(f"[noalloc] {w} workspace of sdpa_fwd_ex: {n_ws} bytes")
    return ins, o, lse, o_ref, l_ref


def test_noalloc_matches_workspace_entry_point_twice():
    big = Workload("decode_big", 8, 32, 8, 1, 32768, 128, "bf16", "bf16", False, 1 / math.sqrt(128), "bshd", 501)
    small = Workload("decode_small", 2, 16, 4, 3, 4096, 128, "bf16", "bf16", True, 1 / math.sqrt(128), "bshd", 502)
    for w in (big, small):
        ins, o, lse, o_ref, l_ref = _both(w)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        heads = [(0, 0), (w.b - 1, w.h_q - 1)]
        q, k, v = (f64(ins[n]) for n in ("q", "k", "v"))
        o64, l64 = attention_forward(q, k, v, w.scale, w.causal, heads=heads)
        check_out(f64(o.cpu()), o64, TOL["bf16"], what="noalloc O vs oracle: ")
        m = ~np.isnan(l64)
        assert (np.abs(lse.cpu().numpy()[m] - l64[m]) / np.maximum(1, np.abs(l64[m]))).max() <= 1e-3


def test_noalloc_rejects_partials_beyond_scratch():
    """b2040, h_q 32 / h_kv 1 (MQA), one query row, 512 keys: 2040 full
    32-row blocks in 2 splits need about 2 * 2040 * 32 * 129 * 4 bytes, past
    the 64 MiB scratch."""
    w = Workload("too_big", 2040, 32, 1, 1, 512, 128, "bf16", "bf16", False, 1 / math.sqrt(128), "bshd", 503)
    need = sdpa.fwd_workspace_size(w.b, w.h_q, w.h_kv, w.s_q, w.s_kv, w.d, torch.bfloat16)
    assert need > (64 << 20)
    lib = sdpa.load_library()
    g = {n: torch.zeros(t, dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
         for n, t in (("q", (w.b, w.s_q, w.h_q, w.d)), ("k", (w.b, w.s_kv, w.h_kv, w.d)),
                      ("v", (w.b, w.s_kv, w.h_kv, w.d)))}
    o = torch.empty_like(g["q"])
    lse = torch.empty((w.b, w.h_q, w.s_q), dtype=torch.float32, device="cuda")
    st = lib.sdpa_fwd_noalloc(*_args(g, o, lse, w), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 2, st  # SDPA_ERR_NOT_SUPPORTED, before any launch
    assert "static scratch" in lib.sdpa_last_error().decode()
