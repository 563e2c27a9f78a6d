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
# dtype (fp16 5e-3, bf16 2e-2, fp8 output 1e-1, fp32 1e-3); LSE
# |err| <= 1e-3 * max(1, |LSE|); gradients at twice the forward's bound.
# Forward outputs are held to the plain max-abs bound. A gradient stored in a
# 16-bit format cannot be closer to the exact value than half a unit in the
# last place of that format: GQA/MQA gradients summed over many query heads
# reach |dV| ~ 20, where bf16's own half-ulp (0.0625) exceeds the 4e-2 bound.
# Only for elements whose half-ulp reaches half the bound is the bound applied
# to the error beyond that rounding; every other element gets the plain bound.
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


def bound_err(a: np.ndarray, ref: np.ndarray, dtype: str, tol: float) -> tuple[float, int]:
    """(max over elements of |a - ref| - slack, number of elements given slack).

    slack is half_ulp(ref) of the storage dtype where that reaches tol / 2 (the
    element's own rounding would eat most of the bound), else 0: every other
    element is held to the plain max-abs bound."""
    m = ~np.isnan(ref)
    if not m.any():
        return 0.0, 0
    r, x = ref[m], a[m]
    hu = half_ulp(r, dtype) if dtype in _MANT_BITS else np.zeros_like(r)
    slack = np.where(hu >= tol / 2, hu, 0.0)
    return float((np.abs(x - r) - slack).max()), int((slack > 0).sum())


def check_out(a: np.ndarray, ref: np.ndarray, tol: float, *, grad_dtype: str | None = None, what: str = "") -> float:
    """Assert the max-abs bound; returns the raw max-abs error.

    Forward outputs (grad_dtype None) get the plain bound. Gradients pass their
    storage dtype: elements whose half-ulp reaches tol / 2 are bounded beyond
    that rounding (bound_err), and the count of such elements is printed."""
    raw = max_abs(a, ref)
    if grad_dtype is None:
        say(f"    {what}max|err|={raw:.3e} relF={rel_fro(a, ref):.3e} (bound {tol:g})")
        assert raw <= tol, (what, raw, tol)
        return raw
    err, n_relaxed = bound_err(a, ref, grad_dtype, tol)
    say(f"    {what}max|err|={raw:.3e} bounded={err:.3e} relaxed_elems={n_relaxed} relF={rel_fro(a, ref):.3e} "
        f"max|ref|={np.nanmax(np.abs(ref)) if ref.size else 0:.2f} (bound {tol:g})")
    assert err <= tol, (what, raw, err, n_relaxed, tol)
    return raw


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    m = ~np.isnan(b)
    return float(np.abs(a[m] - b[m]).max()) if m.any() else 0.0


def check_lse(lse_gpu: np.ndarray, lse_ref: np.ndarray):
    m = ~np.isnan(lse_ref)
    err = np.abs(lse_gpu[m] - lse_ref[m]) / np.maximum(1.0, np.abs(lse_ref[m]))
    assert err.max() <= LSE_REL, f"LSE rel err {err.max():.3e}"
    return float(err.max())


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    """||a - b||_F / ||b||_F over the non-NaN reference entries (0 when both are
    zero, ||a - b||_F when only the reference is)."""
    m = ~np.isnan(b)
    num = float(np.linalg.norm(a[m] - b[m]))
    den = float(np.linalg.norm(b[m]))
    if den == 0.0:
        return num
    return num / den
