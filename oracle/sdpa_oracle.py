"""CPU oracle for scaled dot-product attention, forward and backward, in float64.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module; only the tests, the package smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library: it is the
plain definition written out with numpy, slow and obviously correct.

Sources, by page (the pages are the authority on what is computed):

* The JAX attention codelab ("Speed up attention on GPU with cuDNN and
  TransformerEngine"), step 1 "how attention works": the formula
  softmax(Q K^T / sqrt(d_k)) V and its four steps (scores, scale + softmax,
  weights times V, output of Q's shape). Step 4 "attention from scratch":
  the dense, materialised form this module follows.
* Same codelab, step 7 "add a causal mask": each position attends only to
  itself and earlier positions (lower-triangular mask).
* Same codelab, step 9 "MHA, GQA, MQA": K/V carry fewer heads; each KV head is
  shared by a contiguous group of query heads (read: kv = hq // (h_q / h_kv)).
* The cuDNN 9 blog ("Accelerating Transformers with NVIDIA cuDNN 9"),
  "SDPA as a cuDNN graph" (Figure 4) and the C++ block of "SDPA usage":
  attn_scale multiplies the first matmul's output before the mask and softmax;
  the SDPA node also returns ``stats`` for training.
* Same codelab, step 10 "FP8 path": E4M3 (4 exponent bits, 3 mantissa bits)
  in the forward pass.

Readings where the pages are silent (each one is listed with its reason in the
design notes of the repository):

* ``stats`` is the natural-log logsumexp of the scaled, masked scores of each
  query row: LSE_i = m_i + ln(sum_j exp(S_ij - m_i)), m_i = max_j S_ij.
* the causal mask is top-left aligned by default: key j is visible to query i
  iff j <= i, also when s_q != s_kv. Bottom-right alignment (the option the
  cuDNN 9 blog's SDPA node call lists next to the padding mask) shifts the
  diagonal to the end of the key range: j <= i + (s_kv - s_q).
* the padding mask (the node's ``use_padding_mask`` with per-batch
  ``seq_len_q`` / ``seq_len_kv``): batch element b uses only its first
  seq_len_q[b] query rows and first seq_len_kv[b] keys; the bottom-right
  offset uses those lengths. A query row that sees no key (a padded row, or a
  row above a bottom-right diagonal) has O = 0 and LSE = -inf and takes no
  part in the backward (its dQ is 0 and it adds nothing to dK, dV).
* score modifiers (the node's ``bias`` and ``use_alibi_mask`` options, also
  without semantics on the pages): an additive bias B[b, h, i, j] and an
  ALiBi term -slope[h] * |i + off - j| (off as for the causal diagonal, 0
  without a causal mask) are added to the scaled scores before the mask and
  the softmax; the bias is a constant (no gradient is formed for it).
* the backward is the exact gradient of the forward (the pages only show that
  a forward+backward exists), with D_i = sum_d dO_id * O_id.
* fp8 inputs are the e4m3 codes times a per-tensor fp32 descale; the oracle
  does not quantise P (exact softmax), so the fp8 kernel's P rounding is what
  the fp8 tolerance absorbs.

Memory: rows of queries are processed in blocks so that a (block x s_kv)
score matrix, not (s_q x s_kv), is live. Each row's softmax still spans all of
its keys; for the backward, dK and dV are summed over query blocks (the same
sum, re-associated) — no other reordering.
"""
from __future__ import annotations

import math

import numpy as np

_ROW_BLOCK = 512


def _kv_head(hq: int, h_q: int, h_kv: int) -> int:
    """KV head read by query head hq: contiguous groups of h_q / h_kv query heads."""
    if h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    return hq // (h_q // h_kv)


def _lengths(bi: int, s_q: int, s_kv: int, causal: bool, align: str, seq_len_q, seq_len_kv):
    """(valid query rows, valid keys, diagonal offset) of batch element bi.

    Key j is visible to query row i < lq iff j < lk and, under the causal mask,
    j <= i + off, with off = 0 (top-left) or lk - lq (bottom-right).
    """
    if align not in ("top_left", "bottom_right"):
        raise ValueError("align must be 'top_left' or 'bottom_right'")
    lq = s_q if seq_len_q is None else int(min(max(int(seq_len_q[bi]), 0), s_q))
    lk = s_kv if seq_len_kv is None else int(min(max(int(seq_len_kv[bi]), 0), s_kv))
    off = lk - lq if (causal and align == "bottom_right") else 0
    return lq, lk, off


def _masked_scores(q_rows: np.ndarray, row_idx: np.ndarray, kh: np.ndarray, scale: float,
                   causal: bool, lq: int = None, lk: int = None, off: int = 0, bias_rows=None,
                   slope: float = None) -> np.ndarray:
    """S = scale * Q K^T (+ bias + ALiBi) for the given query rows, with masked
    entries set to -inf.

    bias_rows: optional additive bias for these rows (n_rows x n_keys).
    slope: optional ALiBi slope of this head: adds -slope * |i + off - j|.
    Masked: keys j >= lk, every key of a row i >= lq, and (causal) j > i + off.
    """
    s = scale * (q_rows @ kh.T)
    key_idx = np.arange(kh.shape[0])
    if bias_rows is not None:
        s = s + bias_rows
    if slope is not None:
        s = s - slope * np.abs(row_idx[:, None] + off - key_idx[None, :])
    lq = np.iinfo(np.int64).max if lq is None else lq
    lk = kh.shape[0] if lk is None else lk
    vis = (key_idx[None, :] < lk) & (row_idx[:, None] < lq)
    if causal:
        vis &= key_idx[None, :] <= row_idx[:, None] + off
    return np.where(vis, s, -np.inf)


def _softmax_rows(s: np.ndarray):
    """Row softmax of S: returns (P, m, l) with P = exp(S - m) / l.

    A row whose entries are all -inf (no visible key) gets P = 0, m = -inf and
    l = 0, so that O = 0 and LSE = m + ln l = -inf.
    """
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)
    l = e.sum(axis=1, keepdims=True)
    p = e / np.where(l > 0, l, 1.0)
    return p, np.where(empty, -np.inf, m[:, 0]), l[:, 0]


def _bias_rows(bias, bi, hq, ridx, lk):
    """Rows ridx of the additive bias of (bi, hq), keys < lk; bias is
    (b or 1, h or 1, s_q, s_kv) and broadcasts over its size-1 dims."""
    if bias is None:
        return None
    bb = bias[bi if bias.shape[0] > 1 else 0, hq if bias.shape[1] > 1 else 0]
    return np.asarray(bb[ridx, :lk], dtype=np.float64)


def attention_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      causal: bool, heads=None, rows=None, row_block: int = _ROW_BLOCK,
                      seq_len_q=None, seq_len_kv=None, align: str = "top_left", bias=None,
                      alibi_slopes=None, dropout_p: float = 0.0, dropout_seed: int = 0,
                      dropout_offset: int = 0):
    """Forward pass O = softmax(scale * Q K^T + mask) V and LSE, in float64.

    Follows the JAX attention codelab's step 1 formula and step 4 dense form
    (scores, scale, row softmax, weights times V), with step 7's causal mask,
    step 9's KV-head groups and the ``stats`` output of the cuDNN 9 blog's
    SDPA node (read as the natural-log logsumexp of each row).

    q: (b, h_q, s_q, d); k, v: (b, h_kv, s_kv, d), any real dtype (cast to float64).
    heads: optional list of (b, hq) pairs to compute (default: all).
    rows: optional array of query-row indices to compute (default: all).
    seq_len_q, seq_len_kv: optional per-batch valid lengths (padding mask),
    clamped to [0, s_q] and [0, s_kv]; align: "top_left" or "bottom_right"
    placement of the causal diagonal.
    bias: optional additive bias (b or 1, h_q or 1, s_q, s_kv); alibi_slopes:
    optional per-query-head ALiBi slopes (h_q,).
    dropout_p, dropout_seed, dropout_offset: dropout of the attention weights,
    O = (P * Z) V with Z from ``dropout_mask``; LSE is that of the undropped P.
    Returns (O, LSE): O has shape (b, h_q, n_rows, d) and LSE (b, h_q, n_rows);
    entries for heads not in ``heads`` are NaN. Rows that see no key have
    O = 0 and LSE = -inf.
    """
    b, h_q, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    row_idx_all = np.arange(s_q) if rows is None else np.asarray(rows)
    n = row_idx_all.shape[0]
    out = np.full((b, h_q, n, d), np.nan)
    lse = np.full((b, h_q, n), np.nan)
    pairs = [(bi, hi) for bi in range(b) for hi in range(h_q)] if heads is None else heads
    for bi, hq in pairs:
        g = _kv_head(hq, h_q, h_kv)
        lq, lk, off = _lengths(bi, s_q, s_kv, causal, align, seq_len_q, seq_len_kv)
        kh = np.asarray(k[bi, g, :lk], dtype=np.float64)  # keys past lk are never read
        vh = np.asarray(v[bi, g, :lk], dtype=np.float64)
        for r0 in range(0, n, row_block):
            ridx = row_idx_all[r0:r0 + row_block]
            qr = np.asarray(q[bi, hq][ridx], dtype=np.float64)
            slope = None if alibi_slopes is None else float(alibi_slopes[hq])
            s = _masked_scores(qr, ridx, kh, scale, causal, lq, lk, off, _bias_rows(bias, bi, hq, ridx, lk), slope)
            p, m, l = _softmax_rows(s)
            if dropout_p > 0:
                p = p * dropout_mask(bi * h_q + hq, ridx, lk, dropout_p, dropout_seed, dropout_offset)
            out[bi, hq, r0:r0 + len(ridx)] = p @ vh
            with np.errstate(divide="ignore"):  # ln 0 = -inf for rows that see no key
                lse[bi, hq, r0:r0 + len(ridx)] = m + np.log(l)
    return out, lse


def attention_probs(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
                    seq_len_q=None, seq_len_kv=None, align: str = "top_left", bias=None,
                    alibi_slopes=None) -> np.ndarray:
    """The full attention-weight tensor P (b, h_q, s_q, s_kv); small inputs only.

    The "weights" of the JAX attention codelab's step 1 (rows sum to one; a
    row that sees no key is all zero).
    """
    b, h_q, s_q, _ = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    p_all = np.zeros((b, h_q, s_q, s_kv))
    for bi in range(b):
        lq, lk, off = _lengths(bi, s_q, s_kv, causal, align, seq_len_q, seq_len_kv)
        for hq in range(h_q):
            kh = np.asarray(k[bi, _kv_head(hq, h_q, h_kv), :lk], dtype=np.float64)
            slope = None if alibi_slopes is None else float(alibi_slopes[hq])
            s = _masked_scores(np.asarray(q[bi, hq], dtype=np.float64), np.arange(s_q), kh,
                               scale, causal, lq, lk, off, _bias_rows(bias, bi, hq, np.arange(s_q), lk), slope)
            p_all[bi, hq, :, :lk] = _softmax_rows(s)[0]
    return p_all


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                       scale: float, causal: bool, kv_heads=None, row_block: int = _ROW_BLOCK,
                       seq_len_q=None, seq_len_kv=None, align: str = "top_left", bias=None,
                       alibi_slopes=None, dropout_p: float = 0.0, dropout_seed: int = 0,
                       dropout_offset: int = 0):
    """Gradients (dQ, dK, dV) of L = sum(O * dO) for the forward above, in float64.

    The pages show only that a forward+backward SDPA exists (the cuDNN 9 blog,
    Figure 2); this is the exact gradient of ``attention_forward``, derived by
    the chain rule through the row softmax.

    For each query head hq (KV head g = hq // G), with P the softmax of the
    scaled, masked scores and O = P V:
        D_i  = sum_d dO_id O_id
        dV_g += P^T dO
        dP   = dO V_g^T
        dS   = P * (dP - D[:, None])
        dQ   = scale * dS K_g
        dK_g += scale * dS^T Q
    dK and dV of a KV head are summed over every query head of its group.
    kv_heads: optional list of (b, g) pairs to compute (default: all); the
    other entries are NaN. dQ is filled for the query heads of those groups.
    seq_len_q, seq_len_kv, align: as in ``attention_forward``; rows that see
    no key have P = 0, hence dQ = 0 and no contribution to dK, dV.
    bias, alibi_slopes: as in ``attention_forward``; they only change P.
    dropout_p, dropout_seed, dropout_offset: as in ``attention_forward``; with
    Z the scaled mask, O = (P * Z) V, dV = (P * Z)^T dO, dP = (dO V^T) * Z and
    dS = P * (dP - D), D_i = sum_d dO_id O_id (still equal to sum_j P_ij dP_ij).
    """
    b, h_q, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    grp = h_q // h_kv
    dq = np.full((b, h_q, s_q, d), np.nan)
    dk = np.full((b, h_kv, s_kv, d), np.nan)
    dv = np.full((b, h_kv, s_kv, d), np.nan)
    groups = [(bi, g) for bi in range(b) for g in range(h_kv)] if kv_heads is None else kv_heads
    for bi, g in groups:
        lq, lk, off = _lengths(bi, s_q, s_kv, causal, align, seq_len_q, seq_len_kv)
        kh = np.asarray(k[bi, g, :lk], dtype=np.float64)  # keys past lk are never read
        vh = np.asarray(v[bi, g, :lk], dtype=np.float64)
        dk_g = np.zeros((s_kv, d))
        dv_g = np.zeros((s_kv, d))
        for hq in range(g * grp, (g + 1) * grp):
            assert _kv_head(hq, h_q, h_kv) == g
            qh = np.asarray(q[bi, hq], dtype=np.float64)
            doh = np.asarray(dout[bi, hq], dtype=np.float64)
            dq_h = np.zeros((s_q, d))
            for r0 in range(0, lq, row_block):  # rows past lq are never read; their dQ is 0
                ridx = np.arange(r0, min(lq, r0 + row_block))
                qr, dor = qh[ridx], doh[ridx]
                slope = None if alibi_slopes is None else float(alibi_slopes[hq])
                p, _, _ = _softmax_rows(_masked_scores(qr, ridx, kh, scale, causal, lq, lk, off,
                                                       _bias_rows(bias, bi, hq, ridx, lk), slope))
                z = (dropout_mask(bi * h_q + hq, ridx, lk, dropout_p, dropout_seed, dropout_offset)
                     if dropout_p > 0 else 1.0)
                o = (p * z) @ vh
                dvec = (dor * o).sum(axis=1)
                dv_g[:lk] += (p * z).T @ dor
                dp = (dor @ vh.T) * z
                ds = p * (dp - dvec[:, None])
                dq_h[ridx] = scale * (ds @ kh)
                dk_g[:lk] += scale * (ds.T @ qr)
            dq[bi, hq] = dq_h
        dk[bi, g] = dk_g
        dv[bi, g] = dv_g
    return dq, dk, dv


_PHILOX_M = (0xD2511F53, 0xCD9E8D57)  # round multipliers (Salmon et al. 2011, Philox4x32)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)  # key schedule increments (golden ratio, sqrt(3) - 1)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC 2011), element-wise over uint32 arrays.

    One round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as 64-bit
    products; the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the
    key then advances by (W0, W1) modulo 2^32.
    """
    mask = np.uint64(0xFFFFFFFF)
    c = [np.asarray(x, dtype=np.uint64) & mask for x in (c0, c1, c2, c3)]
    k = [np.asarray(k0, dtype=np.uint64) & mask, np.asarray(k1, dtype=np.uint64) & mask]
    for rnd in range(10):
        if rnd > 0:
            k = [(k[0] + np.uint64(_PHILOX_W[0])) & mask, (k[1] + np.uint64(_PHILOX_W[1])) & mask]
        p0 = np.uint64(_PHILOX_M[0]) * c[0]
        p1 = np.uint64(_PHILOX_M[1]) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return tuple(x.astype(np.uint32) for x in c)


def dropout_keep_threshold(p: float) -> int:
    """k8 = round((1 - p) * 256): an element is kept iff its random byte < k8."""
    return int(min(256, max(0, round((1.0 - float(p)) * 256.0))))


def dropout_mask(bh: int, rows, n_keys: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Scaled dropout mask Z (len(rows) x n_keys) of query head slot bh = b * h_q + h.

    Reading (the SDPA node's ``dropout`` option has no semantics on the pages):
    element (i, j) takes byte (j mod 4) of word (i mod 4) of
    Philox4x32-10(counter = (j // 4, i // 4, bh, offset), key = (seed mod 2^32,
    seed // 2^32)); it is kept iff that byte < k8 = round((1 - p) 256), and a
    kept element is scaled by 256 / k8 (so E[Z] = 1 exactly).
    """
    rows = np.asarray(rows, dtype=np.int64)
    k8 = dropout_keep_threshold(p)
    if k8 == 0:
        return np.zeros((len(rows), n_keys))
    jj = np.arange(n_keys, dtype=np.int64)
    c0 = np.broadcast_to(jj[None, :] >> 2, (len(rows), n_keys))
    c1 = np.broadcast_to(rows[:, None] >> 2, (len(rows), n_keys))
    words = philox4x32_10(c0, c1, np.full(c0.shape, bh), np.full(c0.shape, offset & 0xFFFFFFFF),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(words, axis=0).astype(np.uint64)           # 4 x rows x keys
    sel = w[rows[:, None] % 4, np.arange(len(rows))[:, None], jj[None, :]]
    byte = (sel >> (np.uint64(8) * (jj[None, :] % 4).astype(np.uint64))) & np.uint64(0xFF)
    return np.where(byte < k8, 256.0 / k8, 0.0)


def alibi_slopes(h: int) -> np.ndarray:
    """The ALiBi paper's per-head slopes (Press et al., "Train Short, Test
    Long"): for h a power of two, the geometric sequence 2^(-8/h), 2^(-16/h),
    ..., 2^(-8); otherwise the slopes of the next lower power of two n followed
    by every other slope of 2n."""
    def pow2(n):
        return [2.0 ** (-8.0 * (i + 1) / n) for i in range(n)]
    n = 1 << (h.bit_length() - 1)
    out = pow2(n)
    if n < h:
        out += pow2(2 * n)[0::2][: h - n]
    return np.array(out, dtype=np.float64)


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of OCP e4m3fn codes (uint8) as float64.

    The JAX attention codelab, step 10, names E4M3 (4 exponent bits, 3
    mantissa bits) for the forward pass; the bit layout is the OCP e4m3fn one.

    Layout s eeee mmm, exponent bias 7. e = 0: subnormal (m / 8) * 2^-6.
    e = 15 and m = 7: NaN (the format has no infinities); every other code is
    (1 + m / 8) * 2^(e - 7). Largest finite value 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.power(2.0, e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def fp8_e5m2_decode(codes: np.ndarray) -> np.ndarray:
    """Value of OCP e5m2 codes (uint8) as float64: the gradient format of the
    HYBRID FP8 recipe (JAX attention codelab, step 10: E4M3 in the forward,
    E5M2 in the backward).

    Layout s eeeee mm, exponent bias 15 (IEEE-like). e = 0: subnormal
    (m / 4) * 2^-14; e = 31: infinity (m = 0) or NaN; every other code is
    (1 + m / 4) * 2^(e - 15). Largest finite value 57344.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    normal = (1.0 + m / 4.0) * np.power(2.0, e - 15.0)
    sub = (m / 4.0) * 2.0 ** -14
    val = np.where(e == 0, sub, normal)
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


def fp8_dequantize(codes: np.ndarray, descale: float, fmt: str = "e4m3") -> np.ndarray:
    """Real values x = fp8(code) * descale that an fp8 kernel receives (fmt e4m3 or e5m2)."""
    if fmt == "e5m2":
        return fp8_e5m2_decode(codes) * float(descale)
    return fp8_e4m3_decode(codes) * float(descale)


__all__ = [
    "attention_forward", "attention_backward", "attention_probs", "alibi_slopes", "philox4x32_10",
    "dropout_mask", "dropout_keep_threshold",
    "fp8_e4m3_decode", "fp8_e5m2_decode", "fp8_dequantize",
]

if __name__ == "__main__":  # pragma: no cover - tiny self-demo
    rng = np.random.default_rng(0)
    qq, kk, vv = (rng.standard_normal((1, 2, 4, 3)) for _ in range(3))
    o, l = attention_forward(qq, kk, vv, 1 / math.sqrt(3), True)
    print(o[0, 0], l[0, 0])
