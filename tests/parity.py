"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
on seeded inputs and run the float64 oracle on the very same values."""
from __future__ import annotations

import sys

import numpy as np
import torch

import scaled_dot_product_04_amd as sdpa
import sdpa_inputs
from oracle import attention_backward, attention_forward, fp8_dequantize

# Tolerances: max-abs error of the output vs the float64 oracle, per output
# dtype; LSE |err| <= 1e-3 * max(1, |LSE|); gradients at twice the forward's.
# An output stored in a 16-bit format cannot be closer to the exact value than
# half a unit in the last place of that format, so the bound applied is
# tol + half_ulp(|ref|): for |ref| below 4 (bf16) the extra term is at most
# 0.008, but GQA/MQA gradients summed over many query heads reach 20+, where
# bf16's own rounding (0.0625) exceeds any fixed absolute tolerance.
TOL = {"f32": 1e-3, "f16": 5e-3, "bf16": 2e-2, "fp8": 1e-1}
LSE_REL = 1e-3
_MANT_BITS = {"f32": 23, "f16": 10, "bf16": 7}


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_gpu(ins: dict) -> dict:
    out = {}
    for k, v in ins.items():
        out[k] = sdpa_inputs.to_device_like(v, "cuda") if isinstance(v, torch.Tensor) else v
    return out


def f64(x: torch.Tensor, descale: float | None = None) -> np.ndarray:
    """Exact float64 values of a CPU tensor (fp8 codes times their descale)."""
    if x.dtype == torch.float8_e4m3fn:
        return fp8_dequantize(x.contiguous().view(torch.uint8).numpy(), descale)
    if x.dtype == torch.float8_e5m2:
        return fp8_dequantize(x.contiguous().view(torch.uint8).numpy(), descale, "e5m2")
    return x.double().numpy()


def gpu_fwd(w: sdpa_inputs.Workload, g: dict, return_lse=True, out=None):
    fp8 = None
    if w.dtype == "fp8":
        fp8 = sdpa.Fp8Scales(g["descale_q"], g["descale_k"], g["descale_v"], g["scale_p"], g["descale_p"])
    o, lse = sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=w.causal, fp8=fp8,
                      return_lse=return_lse, out=out)
    torch.cuda.synchronize()
    return o, lse


def oracle_fwd(w, ins, heads=None, rows=None):
    q = f64(ins["q"], ins.get("descale_q"))
    k = f64(ins["k"], ins.get("descale_k"))
    v = f64(ins["v"], ins.get("descale_v"))
    return attention_forward(q, k, v, w.scale, w.causal, heads=heads, rows=rows)


def oracle_bwd(w, ins, kv_heads=None, **kw):
    q, k, v, do = (f64(ins[n], ins.get("descale_" + n)) for n in ("q", "k", "v", "do"))
    return attention_backward(q, k, v, do, w.scale, w.causal, kv_heads=kv_heads, **kw)


def half_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of ``dtype`` at |ref| (normal range)."""
    mag = np.maximum(np.abs(ref), 2.0 ** -14)
    return np.ldexp(1.0, (np.floor(np.log2(mag)) - _MANT_BITS[dtype] - 1).astype(np.int64))


def excess_err(a: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    """max over elements of |a - ref| - half_ulp(ref): the error beyond the output format's rounding."""
    m = ~np.isnan(ref)
    return float((np.abs(a[m] - ref[m]) - half_ulp(ref[m], dtype)).max()) if m.any() else 0.0


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    m = ~np.isnan(b)
    return float(np.abs(a[m] - b[m]).max()) if m.any() else 0.0


def check_lse(lse_gpu: np.ndarray, lse_ref: np.ndarray):
    m = ~np.isnan(lse_ref)
    err = np.abs(lse_gpu[m] - lse_ref[m]) / np.maximum(1.0, np.abs(lse_ref[m]))
    assert err.max() <= LSE_REL, f"LSE rel err {err.max():.3e}"
    return float(err.max())


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    m = ~np.isnan(b)
    return float(np.linalg.norm(a[m] - b[m]) / np.linalg.norm(b[m]))
