"""Seeded synthetic inputs for the attention path and for its CPU oracle.

This module draws random numbers, lays them out in memory (BSHD or BHSD
strides) and rounds them to the I/O dtype. It holds none of the attention
arithmetic, so the HIP path and the oracle can both take their inputs from it
without sharing any of the method.

Recipe (the pages benchmark only random-normal tensors):
  * a ``torch.Generator`` seeded per workload draws fp32 N(0, 1) values in the
    order q, k, v, dO;
  * each tensor is filled in *physical* memory order and then viewed with the
    logical (b, h, s, d) shape through strides, as the "Using cuDNN in Python"
    page does with ``as_strided`` for its BSHD layout;
  * values are rounded (round-to-nearest-even) to the I/O dtype; the GPU and
    the oracle then receive exactly the same bits;
  * fp8-e4m3 inputs are scaled per tensor so that the tensor's largest
    magnitude lands on the format's largest finite value (448), clamped and
    rounded by torch's cast; the fp32 descale factor (1 / scale) travels with
    the bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

FP8_MAX = 448.0  # largest finite OCP e4m3fn value
FP8_E5M2_MAX = 57344.0  # largest finite OCP e5m2 value

_TORCH_DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8": torch.float8_e4m3fn,
}


def physical_shape(b: int, h: int, s: int, d: int, layout: str) -> tuple[int, ...]:
    """Shape of the tensor in memory order for a layout name."""
    if layout == "bshd":
        return (b, s, h, d)
    if layout == "bhsd":
        return (b, h, s, d)
    raise ValueError(f"unknown layout {layout!r}")


def logical_strides(b: int, h: int, s: int, d: int, layout: str) -> tuple[int, int, int, int]:
    """Element strides of the logical (b, h, s, d) view for a layout name."""
    if layout == "bshd":
        return (s * h * d, d, h * d, 1)
    if layout == "bhsd":
        return (h * s * d, s * d, d, 1)
    raise ValueError(f"unknown layout {layout!r}")


def as_logical(phys: torch.Tensor, layout: str) -> torch.Tensor:
    """View a physically laid-out tensor as logical (b, h, s, d) without copying."""
    if layout == "bshd":
        return phys.permute(0, 2, 1, 3)
    return phys


def randn_logical(gen: torch.Generator, b: int, h: int, s: int, d: int,
                  layout: str, dtype: str) -> torch.Tensor:
    """N(0,1) fp32 drawn in physical order, rounded to ``dtype``, viewed as (b,h,s,d)."""
    phys = torch.randn(physical_shape(b, h, s, d, layout), generator=gen, dtype=torch.float32)
    if dtype != "f32":
        phys = phys.to(_TORCH_DTYPES[dtype])
    return as_logical(phys, layout)


def quantize_fp8(x: torch.Tensor, fmt: str = "e4m3") -> tuple[torch.Tensor, float]:
    """Per-tensor fp8 quantisation: returns (fp8 tensor of x's shape/layout, descale).

    scale = fmax / amax(x) (fmax 448 for e4m3, 57344 for e5m2);
    x8 = fp8(clamp(x * scale)); descale = 1 / scale (fp32).
    """
    fmax, tdt = (FP8_E5M2_MAX, torch.float8_e5m2) if fmt == "e5m2" else (FP8_MAX, torch.float8_e4m3fn)
    amax = float(x.abs().max())
    if amax == 0.0:
        amax = 1.0
    scale = fmax / amax
    scaled = (x.float() * scale).clamp_(-fmax, fmax)
    return scaled.to(tdt), float(torch.tensor(1.0 / scale, dtype=torch.float32))


@dataclass
class Workload:
    """One synthetic attention problem."""
    name: str
    b: int
    h_q: int
    h_kv: int
    s_q: int
    s_kv: int
    d: int
    dtype: str            # I/O dtype of q/k/v: f32, f16, bf16 or fp8
    out_dtype: str        # dtype of O (bf16 for fp8 inputs, else the input dtype)
    causal: bool
    scale: float
    layout: str           # "bshd" or "bhsd"
    seed: int
    backward: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def fwd_flops(self) -> float:
        """4*b*h*s_q*s_kv*d, halved under the causal mask."""
        f = 4.0 * self.b * self.h_q * self.s_q * self.s_kv * self.d
        return f / 2 if self.causal else f


def make_inputs(w: Workload, with_grad: bool | None = None) -> dict:
    """Draw q, k, v (and dO when the workload has a backward) on the CPU.

    Returns logical (b, h, s, d) views. For fp8, ``q``/``k``/``v`` are e4m3
    tensors and ``descale_q``/``descale_k``/``descale_v`` hold the factors.
    """
    gen = torch.Generator().manual_seed(w.seed)
    base_dtype = "f32" if w.dtype == "fp8" else w.dtype
    q = randn_logical(gen, w.b, w.h_q, w.s_q, w.d, w.layout, base_dtype)
    k = randn_logical(gen, w.b, w.h_kv, w.s_kv, w.d, w.layout, base_dtype)
    v = randn_logical(gen, w.b, w.h_kv, w.s_kv, w.d, w.layout, base_dtype)
    out = {"q": q, "k": k, "v": v}
    if w.dtype == "fp8":
        for name in ("q", "k", "v"):
            x8, ds = quantize_fp8(out[name])
            out[name] = x8
            out["descale_" + name] = ds
        out["scale_p"] = FP8_MAX
        out["descale_p"] = 1.0 / FP8_MAX
    if with_grad if with_grad is not None else w.backward:
        if w.dtype == "fp8":  # HYBRID: the gradient in e5m2
            do32 = randn_logical(gen, w.b, w.h_q, w.s_q, w.d, w.layout, "f32")
            out["do"], out["descale_do"] = quantize_fp8(do32, "e5m2")
        else:
            out["do"] = randn_logical(gen, w.b, w.h_q, w.s_q, w.d, w.layout, w.out_dtype)
    return out


def make_lengths(b: int, s: int, seed: int, min_len: int = 0) -> torch.Tensor:
    """Per-batch valid lengths for the padding mask: int32 [b], uniform in
    [min_len, s] from a CPU generator seeded with ``seed``; the first entry is
    s (one unpadded batch element) so that full and padded rows both occur."""
    gen = torch.Generator().manual_seed(seed)
    lens = torch.randint(min_len, s + 1, (b,), generator=gen, dtype=torch.int32)
    lens[0] = s
    return lens


def make_bias(shape: tuple, seed: int, dtype: str = "f32") -> torch.Tensor:
    """Additive score bias (b or 1, h or 1, s_q, s_kv): N(0, 1) from a CPU
    generator seeded with ``seed``, rounded to ``dtype``."""
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x.to(_TORCH_DTYPES[dtype])


def empty_logical(b: int, h: int, s: int, d: int, layout: str, dtype: str,
                  device="cpu") -> torch.Tensor:
    """Uninitialised (b, h, s, d) view in ``layout`` (for outputs and gradients)."""
    phys = torch.empty(physical_shape(b, h, s, d, layout), dtype=_TORCH_DTYPES[dtype], device=device)
    return as_logical(phys, layout)


def to_device_like(x: torch.Tensor, device) -> torch.Tensor:
    """Copy a logical view to ``device`` keeping its physical layout (same bytes, same strides)."""
    if x.dim() == 4 and x.stride(3) == 1 and x.stride(1) < x.stride(2):
        # BSHD: the permuted view of a contiguous (b, s, h, d) block
        return x.permute(0, 2, 1, 3).contiguous().to(device).permute(0, 2, 1, 3)
    return x.contiguous().to(device)


# ---------------------------------------------------------------------------
# The workloads. Shapes follow the pages: the GPT-2-like shape of "Using cuDNN
# in Python"; head dim 128 causal and head dim 256 non-causal of the cuDNN 9
# blog's Figures 1-3; MHA/GQA/MQA of the JAX attention codelab (step 9).
# ---------------------------------------------------------------------------

def tiny(causal: bool = False) -> Workload:
    return Workload("tiny_fp32", 1, 2, 2, 128, 128, 64, "f32", "f32", causal,
                    1.0 / math.sqrt(64), "bhsd", 0)


def gpt2() -> Workload:
    return Workload("gpt2_fp16", 4, 12, 12, 1024, 1024, 64, "f16", "f16", True,
                    1.0 / 8.0, "bshd", 0xDEADBEEF)


HD128_SEQS = (512, 1024, 2048, 4096, 8192, 16384)


def hd128(s: int) -> Workload:
    b = 16384 // s
    return Workload(f"hd128_causal_s{s}", b, 16, 16, s, s, 128, "bf16", "bf16", True,
                    1.0 / math.sqrt(128), "bshd", s, backward=True)


def gqa(h_kv: int) -> Workload:
    return Workload(f"gqa_hkv{h_kv}", 2, 32, h_kv, 4096, 4096, 128, "bf16", "bf16", True,
                    1.0 / math.sqrt(128), "bshd", 42 + h_kv, backward=True)


def fp8_hd128() -> Workload:
    """The hd128 causal training shape with fp8 tensors (e4m3) and an e5m2
    gradient, the HYBRID recipe of the JAX attention codelab (step 10)."""
    return Workload("fp8_hd128_causal_s8192", 2, 16, 16, 8192, 8192, 128, "fp8", "bf16", True,
                    1.0 / math.sqrt(128), "bshd", 9128, backward=True)


def fp8() -> Workload:
    return Workload("fp8_hd256", 4, 8, 8, 8192, 8192, 256, "fp8", "bf16", False,
                    1.0 / 16.0, "bshd", 9000)


def kv_cache() -> Workload:
    """One new token per sequence against a 32768-entry KV cache, GQA 32/8
    (the inference use of shared KV heads in the JAX attention codelab,
    step 9); with one query row the causal mask removes nothing."""
    return Workload("kv_cache_decode", 8, 32, 8, 1, 32768, 128, "bf16", "bf16", False, 1 / math.sqrt(128),
                    "bshd", 32768)


def varlen() -> Workload:
    """A ragged batch for the padding mask: 8 sequences padded to 8192 rows,
    h16 d128 bf16, causal; the valid lengths come from make_lengths(8, 8192, 8192)."""
    return Workload("varlen_hd128", 8, 16, 16, 8192, 8192, 128, "bf16", "bf16", True, 1 / math.sqrt(128),
                    "bshd", 8192)


def all_workloads() -> list[Workload]:
    return ([tiny(False), tiny(True), gpt2()] + [hd128(s) for s in HD128_SEQS]
            + [gqa(h) for h in (32, 8, 1)] + [fp8()])
