"""Thin Python binding of libsdpa.so: fused scaled dot-product attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libsdpa.so (declared in include/sdpa.h). torch provides device
memory and the stream. Tensors are logical (b, h, s, d) views with any
strides whose last (d) stride is 1 — e.g. the BSHD layout of "Using cuDNN in
Python", (s*h*d, d, h*d, 1) — and they are passed as pointer + strides
without copies.

If libsdpa.so has not been built this module raises on first use: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa.so")

SDPA_F32, SDPA_F16, SDPA_BF16, SDPA_FP8_E4M3, SDPA_FP8_E5M2 = 0, 1, 2, 3, 4
SDPA_MASK_NONE, SDPA_MASK_CAUSAL, SDPA_MASK_CAUSAL_BOTTOM_RIGHT = 0, 1, 2
STATUS_NAMES = {0: "SDPA_OK", 1: "SDPA_ERR_INVALID_ARGUMENT", 2: "SDPA_ERR_NOT_SUPPORTED",
                3: "SDPA_ERR_WORKSPACE_TOO_SMALL", 4: "SDPA_ERR_HIP"}

_DTYPE_CODES = {torch.float32: SDPA_F32, torch.float16: SDPA_F16, torch.bfloat16: SDPA_BF16,
                torch.float8_e4m3fn: SDPA_FP8_E4M3, torch.float8_e5m2: SDPA_FP8_E5M2}

_Strides = ctypes.c_int64 * 4


class Fp8Scales(ctypes.Structure):
    """sdpa_fp8_scales_t: per-tensor fp8 factors (x = e4m3 code value * descale)."""
    _fields_ = [("descale_q", ctypes.c_float), ("descale_k", ctypes.c_float),
                ("descale_v", ctypes.c_float), ("scale_p", ctypes.c_float),
                ("descale_p", ctypes.c_float)]


class Fp8BwdScales(ctypes.Structure):
    """sdpa_fp8_bwd_scales_t: descale factors of the fp8 backward's q, k, v and
    dO, the quantisation scales of P (e4m3) and dS (ds_dtype), and the optional
    device pointer that receives max |dS|."""
    _fields_ = [("descale_q", ctypes.c_float), ("descale_k", ctypes.c_float),
                ("descale_v", ctypes.c_float), ("descale_do", ctypes.c_float),
                ("scale_p", ctypes.c_float), ("scale_ds", ctypes.c_float), ("ds_dtype", ctypes.c_int),
                ("amax_ds", ctypes.c_void_p)]


class ScoreMod(ctypes.Structure):
    """sdpa_score_mod_t: optional ALiBi slopes and additive bias tensor."""
    _fields_ = [("alibi_slopes", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("bias_dtype", ctypes.c_int),
                ("bias_stride", ctypes.c_int64 * 4), ("dropout_p", ctypes.c_float),
                ("dropout_seed", ctypes.c_uint64), ("dropout_offset", ctypes.c_uint32)]


class SdpaError(RuntimeError):
    """A libsdpa call returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libsdpa.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f, i64p = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.POINTER(ctypes.c_int64)
    lib.sdpa_fwd.restype = ctypes.c_int
    lib.sdpa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i64p, i64p, i64p, i64p, f, i, i, i,
                             ctypes.POINTER(Fp8Scales), vp]
    lib.sdpa_fwd_ex.restype = ctypes.c_int
    lib.sdpa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i64p, i64p, i64p, i64p, f, i, vp, vp,
                                ctypes.POINTER(ScoreMod), i, i, ctypes.POINTER(Fp8Scales), vp, ctypes.c_size_t, vp]
    lib.sdpa_fwd_noalloc.restype = ctypes.c_int
    lib.sdpa_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i64p, i64p, i64p, i64p, f, i, vp, vp,
                                     ctypes.POINTER(ScoreMod), i, i, ctypes.POINTER(Fp8Scales), vp]
    lib.sdpa_fwd_workspace_size.restype = ctypes.c_size_t
    lib.sdpa_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.sdpa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.sdpa_bwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    lib.sdpa_bwd.restype = ctypes.c_int
    lib.sdpa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                             i64p, i64p, i64p, i64p, i64p, i64p, i64p, i64p, f, i, i, vp,
                             ctypes.c_size_t, vp]
    lib.sdpa_bwd_ex.restype = ctypes.c_int
    lib.sdpa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                i64p, i64p, i64p, i64p, i64p, i64p, i64p, i64p, f, i, vp, vp,
                                ctypes.POINTER(ScoreMod), i, vp, ctypes.c_size_t, vp]
    lib.sdpa_bwd_fp8.restype = ctypes.c_int
    lib.sdpa_bwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i,
                                 i64p, i64p, i64p, i64p, i64p, i64p, i64p, i64p, f, i, vp, vp,
                                 i, ctypes.POINTER(Fp8BwdScales), vp, ctypes.c_size_t, vp]
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_status_string.argtypes = [i]
    lib.sdpa_alibi_slopes.restype = ctypes.c_int
    lib.sdpa_mfma_probe.restype = ctypes.c_int
    lib.sdpa_mfma_probe.argtypes = [i, i, i, vp, vp]
    lib.sdpa_alibi_slopes.argtypes = [i, ctypes.POINTER(ctypes.c_float)]
    lib.sdpa_set_timing_events.restype = ctypes.c_int
    lib.sdpa_set_timing_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), i]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().sdpa_last_error().decode()
        raise SdpaError(status, msg)


def _strides(t: torch.Tensor):
    if t.dim() != 4:
        raise ValueError("tensors must be logical (b, h, s, d)")
    return _Strides(*t.stride())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _like_q(q: torch.Tensor, dtype) -> torch.Tensor:
    """An output with q's logical shape and the same physical dim order."""
    order = sorted(range(4), key=lambda dim: -q.stride(dim))
    phys = torch.empty([q.shape[dim] for dim in order], dtype=dtype, device=q.device)
    inv = [order.index(dim) for dim in range(4)]
    return phys.permute(*inv)


def _mask_code(causal) -> int:
    """causal: False / True (top-left) / "top_left" / "bottom_right" -> sdpa_mask_t."""
    if causal is True or causal == "top_left":
        return SDPA_MASK_CAUSAL
    if causal == "bottom_right":
        return SDPA_MASK_CAUSAL_BOTTOM_RIGHT
    if causal is False or causal is None:
        return SDPA_MASK_NONE
    raise ValueError(f"causal must be a bool, 'top_left' or 'bottom_right', not {causal!r}")


def _lens(t, b, device, name):
    """Check a per-batch length tensor (device int32 [b]) and return its pointer."""
    if t is None:
        return None
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != b or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor of shape ({b},)")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")
    return ctypes.c_void_p(t.data_ptr())


def _score_mod(bias, alibi_slopes, b, h_q, s_q, s_kv, device, dropout=None):
    """Build the sdpa_score_mod_t for an optional bias tensor (b or 1, h_q or 1,
    s_q, s_kv), optional fp32 ALiBi slopes (h_q,) and optional dropout
    (p, seed, offset), or None."""
    if bias is None and alibi_slopes is None and (dropout is None or dropout[0] == 0):
        return None
    m = ScoreMod()
    if dropout is not None:
        m.dropout_p, m.dropout_seed, m.dropout_offset = float(dropout[0]), int(dropout[1]), int(dropout[2])
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or tuple(alibi_slopes.shape) != (h_q,) or \
                not alibi_slopes.is_contiguous() or alibi_slopes.device != device:
            raise ValueError(f"alibi_slopes must be a contiguous float32 tensor of shape ({h_q},) on {device}")
        m.alibi_slopes = alibi_slopes.data_ptr()
    if bias is not None:
        if bias.dim() != 4 or bias.shape[0] not in (1, b) or bias.shape[1] not in (1, h_q) or \
                tuple(bias.shape[2:]) != (s_q, s_kv) or bias.device != device:
            raise ValueError(f"bias must be ({b} or 1, {h_q} or 1, {s_q}, {s_kv}) on {device}")
        st = list(bias.stride())
        for dim in (0, 1):
            if bias.shape[dim] == 1:
                st[dim] = 0
        m.bias = bias.data_ptr()
        m.bias_dtype = _DTYPE_CODES[bias.dtype]
        m.bias_stride = _Strides(*st)
    return m


def alibi_slopes(h: int, device="cuda") -> torch.Tensor:
    """The standard ALiBi slopes of h heads as a float32 tensor on ``device``;
    the library computes them (sdpa_alibi_slopes)."""
    buf = (ctypes.c_float * h)()
    _check(load_library().sdpa_alibi_slopes(int(h), buf))
    return torch.tensor(list(buf), dtype=torch.float32, device=device)


def fwd_workspace_size(b, h_q, h_kv, s_q, s_kv, d, dtype) -> int:
    """Workspace bytes of the split-KV forward for this shape (0: not needed)."""
    return int(load_library().sdpa_fwd_workspace_size(b, h_q, h_kv, s_q, s_kv, d, _DTYPE_CODES[dtype]))


def fwd(q, k, v, *, scale: float, causal=False, out=None, lse=None, return_lse: bool = True,
        fp8: Fp8Scales | None = None, out_dtype=None, seq_len_q=None, seq_len_kv=None, bias=None,
        alibi_slopes=None, dropout_p: float = 0.0, dropout_seed: int = 0, dropout_offset: int = 0,
        workspace=None, split_kv: bool = True, stream=None):
    """O (and LSE) of fused attention. Returns (out, lse); lse is None in inference mode.

    q: (b, h_q, s_q, d); k, v: (b, h_kv, s_kv, d); all on the GPU.
    causal: False, True / "top_left", or "bottom_right" (diagonal through the
    last valid query row and key).
    fp8: factors for e4m3 inputs (then out_dtype defaults to bfloat16).
    seq_len_q, seq_len_kv: optional device int32 [b] valid lengths (padding
    mask); rows that see no key get O = 0 and LSE = -inf.
    bias, alibi_slopes: optional score modifiers added to the scaled scores
    (bias (b or 1, h_q or 1, s_q, s_kv), fp32 or q's dtype; slopes fp32 (h_q,)).
    dropout_p, dropout_seed, dropout_offset: dropout of the attention weights
    (Philox4x32-10 stream; the backward must get the same three values).
    workspace: device uint8 buffer for the split-KV path (few query rows,
    many keys); allocated here when the shape needs one and none is given,
    unless split_kv is False (then no workspace is passed, and shapes whose
    split-KV plan needs one run the row-block kernel).
    """
    lib = load_library()
    b, h_q, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    in_code = _DTYPE_CODES[q.dtype]
    mask = _mask_code(causal)
    lq, lk = _lens(seq_len_q, b, q.device, "seq_len_q"), _lens(seq_len_kv, b, q.device, "seq_len_kv")
    mod = _score_mod(bias, alibi_slopes, b, h_q, s_q, s_kv, q.device,
                     (dropout_p, dropout_seed, dropout_offset))
    if out_dtype is None:
        out_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    if out is None:
        out = _like_q(q, out_dtype)
    if lse is None and return_lse:
        lse = torch.empty((b, h_q, s_q), dtype=torch.float32, device=q.device)
    fp8_arg = ctypes.byref(fp8) if fp8 is not None else None
    if workspace is None and fp8 is None and split_kv:
        n = fwd_workspace_size(b, h_q, h_kv, s_q, s_kv, d, q.dtype) if q.dtype in _DTYPE_CODES else 0
        if n > 0:
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    if (mask == SDPA_MASK_CAUSAL_BOTTOM_RIGHT or lq is not None or lk is not None or workspace is not None
            or mod is not None):
        ws_ptr, ws_n = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
        st = lib.sdpa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, h_q, h_kv, s_q, s_kv, d,
                             _strides(q), _strides(k), _strides(v), _strides(out), float(scale), mask, lq, lk,
                             ctypes.byref(mod) if mod is not None else None, in_code, _DTYPE_CODES[out.dtype],
                             fp8_arg, ws_ptr, ws_n, _stream(stream))
    else:
        st = lib.sdpa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, h_q, h_kv, s_q, s_kv, d,
                          _strides(q), _strides(k), _strides(v), _strides(out), float(scale), mask,
                          in_code, _DTYPE_CODES[out.dtype], fp8_arg, _stream(stream))
    _check(st)
    return out, lse


def bwd_workspace_size(b, h_q, h_kv, s_q, s_kv, d, causal, dtype) -> int:
    return int(load_library().sdpa_bwd_workspace_size(b, h_q, h_kv, s_q, s_kv, d, int(causal),
                                                      _DTYPE_CODES[dtype]))


def bwd(q, k, v, o, dout, lse, *, scale: float, causal=False, dq=None, dk=None, dv=None,
        workspace=None, seq_len_q=None, seq_len_kv=None, bias=None, alibi_slopes=None,
        dropout_p: float = 0.0, dropout_seed: int = 0, dropout_offset: int = 0, stream=None):
    """(dQ, dK, dV) of L = sum(O * dO). dK/dV are summed over each KV head's query group.

    causal, seq_len_q, seq_len_kv, bias, alibi_slopes, dropout_*: those of the
    forward that produced o and lse.
    """
    lib = load_library()
    b, h_q, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    mask = _mask_code(causal)
    lq, lk = _lens(seq_len_q, b, q.device, "seq_len_q"), _lens(seq_len_kv, b, q.device, "seq_len_kv")
    mod = _score_mod(bias, alibi_slopes, b, h_q, s_q, s_kv, q.device,
                     (dropout_p, dropout_seed, dropout_offset))
    dq = _like_q(q, q.dtype) if dq is None else dq
    dk = _like_q(k, k.dtype) if dk is None else dk
    dv = _like_q(v, v.dtype) if dv is None else dv
    if workspace is None:
        n = bwd_workspace_size(b, h_q, h_kv, s_q, s_kv, d, mask != SDPA_MASK_NONE, q.dtype)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            b, h_q, h_kv, s_q, s_kv, d, _strides(q), _strides(k), _strides(v), _strides(o),
            _strides(dout), _strides(dq), _strides(dk), _strides(dv), float(scale))
    tail = (_DTYPE_CODES[q.dtype], _ptr(workspace), workspace.numel(), _stream(stream))
    if mask == SDPA_MASK_CAUSAL_BOTTOM_RIGHT or lq is not None or lk is not None or mod is not None:
        st = lib.sdpa_bwd_ex(*args, mask, lq, lk, ctypes.byref(mod) if mod is not None else None, *tail)
    else:
        st = lib.sdpa_bwd(*args, mask, *tail)
    _check(st)
    return dq, dk, dv


def bwd_fp8(q, k, v, o, dout, lse, *, scale: float, descale_q: float, descale_k: float,
            descale_v: float, descale_do: float, scale_ds: float, scale_p: float = 448.0,
            ds_dtype=torch.float8_e4m3fn, amax_ds=None, causal=False, dq=None, dk=None, dv=None,
            workspace=None, seq_len_q=None, seq_len_kv=None, stream=None):
    """(dQ, dK, dV) in bf16 for the fp8 forward: q, k, v e4m3, dout e5m2 (or e4m3),
    o the forward's bf16 output, lse its LSE; real values are code * descale.

    scale_p: P is quantised to e4m3 as P * scale_p (0 < scale_p <= 448).
    scale_ds, ds_dtype: dS is quantised to ds_dtype (float8_e4m3fn or
    float8_e5m2) as dS * scale_ds, saturating.
    amax_ds: optional device float32 tensor of one element; receives
    max(amax_ds, max |dS|) (the caller's scale history input).
    causal, seq_len_q, seq_len_kv: those of the forward that produced o and lse.
    """
    lib = load_library()
    b, h_q, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    mask = _mask_code(causal)
    lq, lk = _lens(seq_len_q, b, q.device, "seq_len_q"), _lens(seq_len_kv, b, q.device, "seq_len_kv")
    if dout.dtype not in (torch.float8_e5m2, torch.float8_e4m3fn):
        raise TypeError(f"dout must be float8_e5m2 or float8_e4m3fn, got {dout.dtype}")
    dq = _like_q(q, torch.bfloat16) if dq is None else dq
    dk = _like_q(k, torch.bfloat16) if dk is None else dk
    dv = _like_q(v, torch.bfloat16) if dv is None else dv
    if workspace is None:
        n = bwd_workspace_size(b, h_q, h_kv, s_q, s_kv, d, mask != SDPA_MASK_NONE, torch.float8_e4m3fn)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    if ds_dtype not in (torch.float8_e5m2, torch.float8_e4m3fn):
        raise TypeError(f"ds_dtype must be float8_e5m2 or float8_e4m3fn, got {ds_dtype}")
    if amax_ds is not None and (amax_ds.dtype != torch.float32 or amax_ds.numel() < 1 or not amax_ds.is_cuda):
        raise TypeError("amax_ds must be a float32 device tensor with at least one element")
    sc = Fp8BwdScales(float(descale_q), float(descale_k), float(descale_v), float(descale_do), float(scale_p),
                      float(scale_ds), _DTYPE_CODES[ds_dtype], amax_ds.data_ptr() if amax_ds is not None else None)
    _check(lib.sdpa_bwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                            _ptr(dv), b, h_q, h_kv, s_q, s_kv, d, _strides(q), _strides(k), _strides(v),
                            _strides(o), _strides(dout), _strides(dq), _strides(dk), _strides(dv),
                            float(scale), mask, lq, lk, _DTYPE_CODES[dout.dtype], ctypes.byref(sc),
                            _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv


__all__ = ["fwd", "bwd", "bwd_fp8", "Fp8BwdScales", "SDPA_FP8_E5M2", "bwd_workspace_size", "fwd_workspace_size", "alibi_slopes", "ScoreMod", "load_library", "library_path", "Fp8Scales",
           "SdpaError", "SDPA_F32", "SDPA_F16", "SDPA_BF16", "SDPA_FP8_E4M3", "SDPA_MASK_NONE",
           "SDPA_MASK_CAUSAL", "SDPA_MASK_CAUSAL_BOTTOM_RIGHT"]
