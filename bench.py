#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X.

One step = one forward (O, LSE) and one backward (dQ, dK, dV) of causal
scaled dot-product attention with head dim 128 in bf16, on the s=8192 point of
the head-dim-128 sweep (b=2, h=16, b*s = 16384 tokens, BSHD layout), all
inputs resident in HBM. The reported value is TFLOP/s of the whole step under
the counting 4*b*h*s_q*s_kv*d per forward (halved under the causal mask) and
2.5x that per backward, as in the cuDNN 9 blog's forward and forward+backward
figures (Figures 1 and 2). GPU time only (events on the launch stream), the
convention the blog states for its measurements.

Prints one JSON line on stdout. Also reports:
  * roofline: the dominant kernel's achieved TFLOP/s (its own matmul flops per
    launch / its mean duration from events recorded around it inside the
    library) against the MI355X dense bf16 MFMA peak;
  * cpu_baseline: the float64 CPU oracle timed on a bounded sample of the same
    workload (a few (b, h) heads, forward + backward) on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls needed to time kernels with events."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return float(out.value)


def cpu_baseline(w, ins, n_heads: int) -> dict:
    """Time the float64 oracle (as it stands) on n_heads (b, h) heads, fwd + bwd."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_backward, attention_forward

    heads = [(0, h) for h in range(n_heads)]
    # only the sampled heads are converted to float64
    q = np.stack([ins["q"][0, h].double().numpy() for _, h in heads])[None]
    k = np.stack([ins["k"][0, h].double().numpy() for _, h in heads])[None]
    v = np.stack([ins["v"][0, h].double().numpy() for _, h in heads])[None]
    do = np.stack([ins["do"][0, h].double().numpy() for _, h in heads])[None]
    t0 = time.perf_counter()
    attention_forward(q, k, v, w.scale, w.causal)
    attention_backward(q, k, v, do, w.scale, w.causal)
    dt = time.perf_counter() - t0
    flops = 3.5 * 4.0 * n_heads * w.s_q * w.s_kv * w.d / (2 if w.causal else 1)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_heads} of {w.b * w.h_q} (b, h) heads of the same workload, forward + backward, "
                      f"float64 numpy; {dt:.2f} s wall",
            "seconds": round(dt, 3)}


TRAFFIC_RECORDS = {"bwd_dkdv": "profiles/hd128_causal_s8192_dkdv_hbm_traffic.json",
                   "fwd": "profiles/hd128_causal_s8192_fwd_hbm_traffic.json",
                   "bwd_dq": "profiles/hd128_causal_s8192_dq_hbm_traffic.json"}


def kernel_sources(kernel: str) -> list:
    """Files whose content decides what `kernel` does: its kernel file, the
    shared device helpers, the argument layouts and variant levels, the build
    flags. A traffic record counts only while all of them are unchanged."""
    csrc = "scaled_dot_product_04_amd/csrc/"
    main = csrc + ("bwd_kernels.hip" if kernel.startswith("bwd") else "fwd_kernels.hip")
    return [main, csrc + "device_common.h", csrc + "sdpa_internal.h", "scaled_dot_product_04_amd/_build.py"]


def sources_digest(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter record
    (FETCH_SIZE and WRITE_SIZE, scaled by a known-size copy), or None when there
    is no record or the kernel's sources changed since the counters were taken."""
    import json
    rec_path = TRAFFIC_RECORDS.get(kernel)
    if rec_path is None or not os.path.exists(os.path.join(ROOT, rec_path)):
        return None
    rec = json.load(open(os.path.join(ROOT, rec_path)))
    if rec.get("sources") != kernel_sources(kernel) or sources_digest(kernel_sources(kernel)) != rec["sources_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def write_traffic_record(kernel: str, fetch_db: str, write_db: str, copy_fetch_db: str, copy_write_db: str,
                         commands: list) -> str:
    """Build the committed HBM-traffic record of one kernel from four rocprofv3
    --pmc result databases (FETCH_SIZE and WRITE_SIZE of a bench run, and of
    `bench.py --copy-reference`). Each counter is averaged per dispatch and
    scaled so that the 1 GiB copy reads 1 GiB and writes 1 GiB. No GPU use."""
    import json
    import sqlite3

    short = {"bwd_dkdv": "bwd_dkdv64_kernel<sdpa::Bf16T, true>",
             "fwd": "fwd_mfma_kernel<sdpa::Bf16T, 128, true, 8, 0, 1>",
             "bwd_dq": "bwd_dq_kernel<sdpa::Bf16T, 128, true, 0>"}[kernel]

    def per_dispatch(db, counter, name_part=None):
        c = sqlite3.connect(db)
        tot = {}
        for kn, cn, did, v in c.execute("select kernel_name, counter_name, dispatch_id, value from counters_collection"):
            if cn == counter and (name_part is None or name_part in kn):
                tot.setdefault((kn, did), 0.0)
                tot[(kn, did)] += v
        if name_part is None:  # the copy run: the kernel that moved the most bytes
            best = max({k[0] for k in tot}, key=lambda n: sum(v for k, v in tot.items() if k[0] == n))
            tot = {k: v for k, v in tot.items() if k[0] == best}
        return sum(tot.values()) / len(tot)

    gib_kib = float(1 << 20)
    fetch_scale = gib_kib / per_dispatch(copy_fetch_db, "FETCH_SIZE")
    write_scale = gib_kib / per_dispatch(copy_write_db, "WRITE_SIZE")
    fetch = per_dispatch(fetch_db, "FETCH_SIZE", short)
    write = per_dispatch(write_db, "WRITE_SIZE", short)
    sources = kernel_sources(kernel)
    rec = {"kernel": short, "workload": "hd128_causal_s8192 (b2 h16 s8192 d128 bf16 causal BSHD)",
           "fetch_size_kib_per_launch": round(fetch, 1), "write_size_kib_per_launch": round(write, 1),
           "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
           "hbm_bytes_per_launch": int(round((fetch * fetch_scale + write * write_scale) * 1024)),
           "commands": commands, "sources": sources, "sources_sha256": sources_digest(sources)}
    out = TRAFFIC_RECORDS[kernel]
    with open(os.path.join(ROOT, out), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return out


def _short_kernel(name: str) -> str:
    import re
    m = re.search(r"(\w+_kernel)(<[^()]*>)?", name)
    return (m.group(1) + (m.group(2) or "")).replace("sdpa::", "") if m else name[:60]


def summarize_trace(db: str, last: int = 0) -> str:
    """Markdown table of a rocprofv3 --kernel-trace result database: per kernel,
    launches, total, mean and median duration (us); with last > 0 also the mean
    of the last `last` launches of each kernel (the timed steps after warm-up).
    No GPU use."""
    import sqlite3
    c = sqlite3.connect(db)
    per = {}
    for name, start, end in c.execute("select name, start, end from kernels"):
        per.setdefault(_short_kernel(name), []).append((start, (end - start) / 1000.0))
    total = sum(d for v in per.values() for _, d in v)
    lines = ["| kernel | launches | total us | mean us | median us | % of GPU time |"
             + (f" mean of last {last} us |" if last else ""),
             "|---|---|---|---|---|---|" + ("---|" if last else "")]
    for k, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        d = [x for _, x in sorted(v)]
        row = (f"| `{k}` | {len(d)} | {sum(d):.1f} | {statistics.fmean(d):.1f} | {statistics.median(d):.1f} | "
               f"{100 * sum(d) / total:.1f} |")
        if last:
            row += f" {statistics.fmean(d[-last:]):.1f} |"
        lines.append(row)
    return "\n".join(lines)


def summarize_counters(dbs: list) -> str:
    """Markdown table of rocprofv3 --pmc result databases: per kernel, the
    median per dispatch of every counter collected, and where the counters
    allow it the derived clock (GRBM_GUI_ACTIVE per XCD over the dispatch
    duration) and MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over
    1024 SIMDs x clock x duration). No GPU use."""
    import sqlite3
    per = {}
    for db in dbs:
        c = sqlite3.connect(db)
        for kn, cn, did, v, dur in c.execute(
                "select kernel_name, counter_name, dispatch_id, value, duration from counters_collection"):
            k = _short_kernel(kn)
            ent = per.setdefault(k, {}).setdefault((db, did), {"dur": dur})
            ent[cn] = ent.get(cn, 0.0) + v
    out = []
    for k, disp in sorted(per.items()):
        vals = {}
        for ent in disp.values():
            for cn, v in ent.items():
                vals.setdefault(cn, []).append(v)
        med = {cn: statistics.median(v) for cn, v in vals.items()}
        out.append(f"`{k}` ({len(disp)} dispatch records)")
        out.append("")
        out.append("| counter | median per dispatch |")
        out.append("|---|---|")
        for cn in sorted(med):
            if cn != "dur":
                out.append(f"| {cn} | {med[cn]:.6g} |")
        # Rates per dispatch record (counter / that record's duration), then medians.
        def rate(cn, div):
            r = [e[cn] / div / (e["dur"] / 1e9) for e in disp.values() if cn in e and e["dur"] > 0]
            return statistics.median(r) if r else None
        clk = rate("GRBM_GUI_ACTIVE", 8)
        if clk is not None:
            out.append(f"| clock: GRBM_GUI_ACTIVE / 8 XCDs / duration | {clk / 1e9:.2f} GHz |")
        clk2 = rate("SQ_CYCLES", 32)
        if clk2 is not None:
            out.append(f"| clock: SQ_CYCLES / 32 SEs / duration | {clk2 / 1e9:.2f} GHz |")
        busy = rate("SQ_VALU_MFMA_BUSY_CYCLES", 1024)
        if busy is not None and (clk or clk2):
            f = clk or clk2
            out.append(f"| MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x clock x duration) | "
                       f"{100 * busy / f:.1f} % |")
            out.append(f"| same, against the 2.4 GHz clock of the published peak | {100 * busy / 2.4e9:.1f} % |")
        out.append("")
    return "\n".join(out)


def mfma_measured(sdpa, torch, hip, stream, sh) -> dict:
    """Sustained dense MFMA rate (bf16 32x32x16, fp8 32x32x64) and the shader
    clock while the matrix pipes are saturated, from the library's rate probe
    (sdpa_mfma_probe): the measured denominator beside the published peaks."""
    lib = sdpa.load_library()
    blocks = 2 * 256  # two 4-wave workgroups per CU: two waves on every SIMD
    stamps = torch.zeros(4 * blocks, dtype=torch.int64, device="cuda:0")
    out = {}
    for name, code, flops_per in (("bf16", sdpa.SDPA_BF16, 32768.0), ("fp8", sdpa.SDPA_FP8_E4M3, 131072.0)):
        iters = 40000 if name == "bf16" else 20000
        best = None
        for rep in range(4):  # the first launch warms up; keep the fastest of the rest
            a, b = hip.event(), hip.event()
            hip.record(a, sh)
            st = lib.sdpa_mfma_probe(code, blocks, iters, ctypes.c_void_p(stamps.data_ptr()), sh)
            hip.record(b, sh)
            if st != 0:
                raise RuntimeError(lib.sdpa_last_error().decode())
            torch.cuda.synchronize()
            ms = hip.ms(a, b)
            if rep > 0 and (best is None or ms < best[0]):
                s = stamps.view(blocks, 4).cpu().double()
                cycles, real = s[:, 1] - s[:, 0], s[:, 3] - s[:, 2]
                clk = float(statistics.median((cycles / real * 0.1).tolist()))  # GHz (real time counts at 100 MHz)
                best = (ms, clk)
                log(f"[bench] probe {name}: {ms:.3f} ms, median cycles {statistics.median(cycles.tolist()):.0f}, "
                    f"median real ticks {statistics.median(real.tolist()):.0f}")
        tf = blocks * 4 * iters * 8 * flops_per / (best[0] / 1e3) / 1e12
        out[f"{name}_tflops"] = round(tf, 1)
        out[f"{name}_clock_ghz"] = round(best[1], 3)
    out["probe"] = "sdpa_mfma_probe: 512 workgroups x 4 waves, 8 independent MFMA chains per wave"
    return out


def fp8_forward(sdpa, sdpa_inputs, torch, hip, stream, sh, warmup: int, steps: int) -> dict:
    """Extra measurement (not part of `value`): the fp8 e4m3 forward on the
    head-dim-256 non-causal workload (b4 h8 s8192), TFLOP/s vs the fp8 peak."""
    w = sdpa_inputs.fp8()
    ins = sdpa_inputs.make_inputs(w)
    g = {k: sdpa_inputs.to_device_like(v, "cuda:0") for k, v in ins.items() if isinstance(v, torch.Tensor)}
    sc = sdpa.Fp8Scales(ins["descale_q"], ins["descale_k"], ins["descale_v"], ins["scale_p"], ins["descale_p"])
    o = sdpa._like_q(g["q"], torch.bfloat16)
    lse = torch.empty((w.b, w.h_q, w.s_q), dtype=torch.float32, device="cuda:0")
    for _ in range(warmup):
        sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=False, out=o, lse=lse, fp8=sc, stream=stream)
    a, b = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(a, sh)
    for _ in range(steps):
        sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=False, out=o, lse=lse, fp8=sc, stream=stream)
    hip.record(b, sh)
    torch.cuda.synchronize()
    ms = hip.ms(a, b) / steps
    tf = w.fwd_flops / (ms / 1e3) / 1e12
    return {"workload": w.name, "ms": round(ms, 4), "tflops": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
            "pct_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2)}


def fp8_hd128_forward_backward(sdpa, sdpa_inputs, torch, hip, stream, sh, warmup: int, steps: int,
                               bf16_ms_step: float) -> dict:
    """Extra measurement (not part of `value`): the hd128 causal training step
    (b2 h16 s8192 d128) with e4m3 tensors and an e5m2 gradient (HYBRID):
    fp8 forward, then the fp8 backward (all five products on fp8 MFMAs, dS in
    e4m3); TFLOP/s of the same counted flops as the bf16 step, and the
    speed-up over it. scale_ds is set the delayed-scaling way before timing:
    one backward with scale 1 reports max |dS|, the timed ones use the power
    of two that maps it inside e4m3."""
    w = sdpa_inputs.fp8_hd128()
    ins = sdpa_inputs.make_inputs(w)
    dev = torch.device("cuda:0")
    g = {k: sdpa_inputs.to_device_like(v, dev) for k, v in ins.items() if isinstance(v, torch.Tensor)}
    sc = sdpa.Fp8Scales(ins["descale_q"], ins["descale_k"], ins["descale_v"], ins["scale_p"], ins["descale_p"])
    o = sdpa._like_q(g["q"], torch.bfloat16)
    lse = torch.empty((w.b, w.h_q, w.s_q), dtype=torch.float32, device=dev)
    dq = sdpa._like_q(g["q"], torch.bfloat16)
    dk, dv = sdpa._like_q(g["k"], torch.bfloat16), sdpa._like_q(g["v"], torch.bfloat16)
    ws = torch.empty(max(16, sdpa.bwd_workspace_size(w.b, w.h_q, w.h_kv, w.s_q, w.s_kv, w.d, True,
                                                     torch.float8_e4m3fn)), dtype=torch.uint8, device=dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    bw = dict(scale=w.scale, causal=True, descale_q=ins["descale_q"], descale_k=ins["descale_k"],
              descale_v=ins["descale_v"], descale_do=ins["descale_do"], dq=dq, dk=dk, dv=dv, workspace=ws,
              stream=stream, scale_ds=1.0, amax_ds=amax)

    def fwd():
        sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=True, out=o, lse=lse, fp8=sc, stream=stream)

    fwd()
    sdpa.bwd_fp8(g["q"], g["k"], g["v"], o, g["do"], lse, **bw)
    torch.cuda.synchronize()
    bw["scale_ds"] = 2.0 ** math.floor(math.log2(448.0 / max(amax.item(), 1e-30)))
    bw["amax_ds"] = None

    def bwd():
        sdpa.bwd_fp8(g["q"], g["k"], g["v"], o, g["do"], lse, **bw)

    res = {"workload": w.name, "b": w.b, "h": w.h_q, "s": w.s_q, "d": w.d,
           "formats": "e4m3 q/k/v/P/dS, e5m2 dO", "scale_ds": bw["scale_ds"]}
    for name, fn in (("forward", fwd), ("backward", bwd), ("step", lambda: (fwd(), bwd()))):
        for _ in range(warmup):
            fn()
        a, b = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(a, sh)
        for _ in range(steps):
            fn()
        hip.record(b, sh)
        torch.cuda.synchronize()
        ms = hip.ms(a, b) / steps
        fl = {"forward": 1.0, "backward": 2.5, "step": 3.5}[name] * w.fwd_flops
        res[name] = {"ms": round(ms, 4), "tflops": round(fl / (ms / 1e3) / 1e12, 2)}
    res["step_speedup_vs_bf16"] = round(bf16_ms_step / res["step"]["ms"], 3)
    return res


def decode_forward(sdpa, sdpa_inputs, torch, hip, stream, sh, warmup: int, steps: int) -> dict:
    """Extra measurement (not part of `value`): a KV-cache step (b8, h_q 32 /
    h_kv 8, one query row, 32768 keys, d128 bf16), bound by HBM: the K/V bytes
    read once per KV head over the time, vs the HBM peak. The row-block kernel
    (which re-reads K/V per query head) is timed beside the split-KV path."""
    w = sdpa_inputs.kv_cache()
    ins = sdpa_inputs.make_inputs(w)
    g = {k: sdpa_inputs.to_device_like(v, "cuda:0") for k, v in ins.items() if isinstance(v, torch.Tensor)}
    o = sdpa._like_q(g["q"], torch.bfloat16)
    lse = torch.empty((w.b, w.h_q, w.s_q), dtype=torch.float32, device="cuda:0")
    n_ws = sdpa.fwd_workspace_size(w.b, w.h_q, w.h_kv, w.s_q, w.s_kv, w.d, torch.bfloat16)
    ws = torch.empty(max(n_ws, 16), dtype=torch.uint8, device="cuda:0")
    res = {"workload": w.name, "b": w.b, "h_q": w.h_q, "h_kv": w.h_kv, "s_q": w.s_q, "s_kv": w.s_kv, "d": w.d}
    kv_bytes = 2 * w.b * w.h_kv * w.s_kv * w.d * 2 + 2 * w.b * w.h_q * w.s_q * w.d * 2 + 4 * w.b * w.h_q * w.s_q
    for name, kw in (("split_kv", {"workspace": ws}), ("row_block", {"split_kv": False})):
        for _ in range(warmup):
            sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=False, out=o, lse=lse, stream=stream, **kw)
        a, b = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(a, sh)
        for _ in range(steps):
            sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=False, out=o, lse=lse, stream=stream, **kw)
        hip.record(b, sh)
        torch.cuda.synchronize()
        ms = hip.ms(a, b) / steps
        gbs = kv_bytes / (ms / 1e3) / 1e9
        res[name] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2)}
    res["algorithmic_bytes"] = kv_bytes
    return res


def varlen_forward_backward(sdpa, sdpa_inputs, torch, hip, stream, sh, warmup: int, steps: int) -> dict:
    """Extra measurement (not part of `value`): forward + backward of a ragged
    batch under the padding mask (8 sequences padded to 8192 rows, h16 d128
    bf16, causal), counted over the valid rows and keys only, next to the same
    padded shape run without lengths (every row counted)."""
    w = sdpa_inputs.varlen()
    lens = sdpa_inputs.make_lengths(w.b, w.s_q, w.seed, min_len=1)
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    dev = torch.device("cuda:0")
    g = {k: sdpa_inputs.to_device_like(v, dev) for k, v in ins.items() if isinstance(v, torch.Tensor)}
    lens_d = lens.to(dev)
    o = torch.empty_like(g["q"])
    lse = torch.empty((w.b, w.h_q, w.s_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
    ws = torch.empty(max(sdpa.bwd_workspace_size(w.b, w.h_q, w.h_kv, w.s_q, w.s_kv, w.d, True, torch.bfloat16), 16),
                     dtype=torch.uint8, device=dev)
    res = {"workload": w.name, "b": w.b, "h": w.h_q, "s_max": w.s_q, "d": w.d, "lengths": lens.tolist()}
    per_head = [4.0 * int(n) * int(n) * w.d / 2 for n in lens]  # causal, square per sequence
    flops_valid = 3.5 * w.h_q * sum(per_head)
    flops_padded = 3.5 * w.fwd_flops
    for name, kw in (("padding_mask", {"seq_len_q": lens_d, "seq_len_kv": lens_d}), ("dense", {})):
        def step():
            sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=True, out=o, lse=lse, stream=stream, **kw)
            sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=True, dq=dq, dk=dk, dv=dv,
                     workspace=ws, stream=stream, **kw)
        for _ in range(warmup):
            step()
        a, b = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(a, sh)
        for _ in range(steps):
            step()
        hip.record(b, sh)
        torch.cuda.synchronize()
        ms = hip.ms(a, b) / steps
        fl = flops_valid if name == "padding_mask" else flops_padded
        res[name] = {"ms": round(ms, 4), "tflops": round(fl / (ms / 1e3) / 1e12, 2),
                     "pct_peak": round(100 * fl / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    res["valid_fraction_of_flops"] = round(flops_valid / flops_padded, 4)
    return res


def config_sweep(sdpa, sdpa_inputs, torch, hip, warmup: int, steps: int) -> list:
    """Full-size timing of every workload the parity tests cover: the hd128
    causal sweep (s = 512 .. 16384, b = 16384 / s), GQA / MQA (h_q 32,
    h_kv 32 / 8 / 1), the GPT-2-like fp16 forward and the fp8 hd256 forward.
    One dict per workload: forward (and forward + backward) ms and TFLOP/s of
    the counted flops, against the dtype's dense peak, after a warm-up of at
    least 0.3 s of the same calls."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    ws = [sdpa_inputs.hd128(s) for s in sdpa_inputs.HD128_SEQS]
    ws += [sdpa_inputs.gqa(h) for h in (32, 8, 1)] + [sdpa_inputs.gpt2(), sdpa_inputs.fp8()]
    out = []
    for w in ws:
        ins = sdpa_inputs.make_inputs(w, with_grad=w.backward)
        g = {k: sdpa_inputs.to_device_like(v, dev) for k, v in ins.items() if isinstance(v, torch.Tensor)}
        fp8 = None
        if w.dtype == "fp8":
            fp8 = sdpa.Fp8Scales(ins["descale_q"], ins["descale_k"], ins["descale_v"], ins["scale_p"],
                                 ins["descale_p"])
        o = sdpa._like_q(g["q"], torch.bfloat16 if w.dtype == "fp8" else g["q"].dtype)
        lse = torch.empty((w.b, w.h_q, w.s_q), dtype=torch.float32, device=dev)
        peak = PEAK_FP8_TFLOPS if w.dtype == "fp8" else PEAK_BF16_TFLOPS
        res = {"workload": w.name, "b": w.b, "h_q": w.h_q, "h_kv": w.h_kv, "s": w.s_q, "d": w.d,
               "dtype": w.dtype, "causal": w.causal}

        def fwd():
            sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=w.causal, out=o, lse=lse, fp8=fp8, stream=stream)

        fns = [("forward", fwd, 1.0)]
        if w.backward:
            dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
            wsp = torch.empty(max(16, sdpa.bwd_workspace_size(w.b, w.h_q, w.h_kv, w.s_q, w.s_kv, w.d, w.causal,
                                                              g["q"].dtype)), dtype=torch.uint8, device=dev)

            def step():
                fwd()
                sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=w.causal, dq=dq, dk=dk,
                         dv=dv, workspace=wsp, stream=stream)
            fns.append(("forward_backward", step, 3.5))
        for name, fn, mult in fns:
            # The GPU clock ramps up over the first ~20 ms of sustained work:
            # warm up for at least 0.3 s as well as `warmup` calls.
            t0, n = time.perf_counter(), 0
            while n < warmup or time.perf_counter() - t0 < 0.3:
                fn()
                n += 1
                if n % 8 == 0:
                    torch.cuda.synchronize()
            a, b = hip.event(), hip.event()
            torch.cuda.synchronize()
            hip.record(a, sh)
            for _ in range(steps):
                fn()
            hip.record(b, sh)
            torch.cuda.synchronize()
            ms = hip.ms(a, b) / steps
            tf = mult * w.fwd_flops / (ms / 1e3) / 1e12
            res[name] = {"ms": round(ms, 4), "tflops": round(tf, 2), "pct_peak": round(100 * tf / peak, 2)}
        log(f"[bench] {res}")
        out.append(res)
        del g, o, lse, ins
        torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The GPU clock ramps up over the first ~100 ms of sustained work: the
    # default warm-up (about 0.14 s of steps) times the kernels at steady clocks.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warmup-s", type=float, default=0.5,
                    help="minimum seconds of warm-up steps before timing (on top of --warmup steps)")
    ap.add_argument("--seq", type=int, default=8192, help="sequence length of the hd128 sweep point (b = 16384/s)")
    ap.add_argument("--cpu-heads", type=int, default=8, help="heads the CPU oracle baseline times (0 = skip)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the extra fp8 forward measurement")
    ap.add_argument("--no-decode", action="store_true", help="skip the extra KV-cache decode measurement")
    ap.add_argument("--no-varlen", action="store_true", help="skip the extra padding-mask (ragged batch) measurement")
    ap.add_argument("--no-mods", action="store_true", help="skip the extra score-modifier (ALiBi, dropout) measurement")
    ap.add_argument("--traffic-record", nargs=5, metavar=("KERNEL", "FETCH_DB", "WRITE_DB", "COPY_FETCH_DB",
                                                          "COPY_WRITE_DB"),
                    help="write the HBM-traffic record of KERNEL from rocprofv3 --pmc result databases and exit "
                         "(no GPU use)")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="print a markdown table of a rocprofv3 --kernel-trace result database and exit (no GPU use)")
    ap.add_argument("--last", type=int, default=0, help="with --summarize-trace: also average the last N launches")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DB",
                    help="print markdown tables of rocprofv3 --pmc result databases and exit (no GPU use)")
    ap.add_argument("--config-sweep", action="store_true",
                    help="time every full-size workload of the parity tests (one JSON object per line) and exit")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the known-size kernel that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings) and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.last))
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return 0
    if args.traffic_record:
        k, f_db, w_db, cf_db, cw_db = args.traffic_record
        cmds = [f"rocprofv3 --pmc FETCH_SIZE -d <out> -o run -- python3 bench.py --steps 2 --warmup 1 --cpu-heads 0 "
                f"--no-fp8 --no-decode --no-varlen --no-mods",
                f"rocprofv3 --pmc WRITE_SIZE -d <out> -o run -- python3 bench.py --steps 2 --warmup 1 --cpu-heads 0 "
                f"--no-fp8 --no-decode --no-varlen --no-mods",
                "rocprofv3 --pmc FETCH_SIZE -d <out> -o run -- python3 bench.py --copy-reference",
                "rocprofv3 --pmc WRITE_SIZE -d <out> -o run -- python3 bench.py --copy-reference",
                f"python3 bench.py --traffic-record {k} <fetch db> <write db> <copy fetch db> <copy write db>"]
        log(f"[bench] wrote {write_traffic_record(k, f_db, w_db, cf_db, cw_db, cmds)}")
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path.", file=sys.stderr)
        return 2
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py is single-process, single-GPU", file=sys.stderr)
        return 2

    import torch

    if args.copy_reference:
        x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        log("[bench] copied 1 GiB five times")
        return 0

    import scaled_dot_product_04_amd as sdpa
    import sdpa_inputs

    if args.config_sweep:
        for res in config_sweep(sdpa, sdpa_inputs, torch, Hip(), args.warmup, args.steps):
            print(json.dumps(res), flush=True)
        return 0

    w = sdpa_inputs.hd128(args.seq)
    log(f"[bench] workload {w.name}: b={w.b} h={w.h_q} s={w.s_q} d={w.d} bf16 causal BSHD")
    ins = sdpa_inputs.make_inputs(w, with_grad=True)
    dev = torch.device("cuda:0")
    g = {k: sdpa_inputs.to_device_like(v, dev) for k, v in ins.items() if isinstance(v, torch.Tensor)}
    o = torch.empty_like(g["q"])
    lse = torch.empty((w.b, w.h_q, w.s_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
    ws = torch.empty(max(16, sdpa.bwd_workspace_size(w.b, w.h_q, w.h_kv, w.s_q, w.s_kv, w.d, w.causal,
                                                     torch.bfloat16)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    lib = sdpa.load_library()
    lib.sdpa_set_timing_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    hip = Hip()

    def step(ev=None):
        if ev is not None:
            lib.sdpa_set_timing_events((ctypes.c_void_p * 2)(*ev[0:2]), 2)
        sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=True, out=o, lse=lse, stream=stream)
        if ev is not None:
            lib.sdpa_set_timing_events((ctypes.c_void_p * 3)(*ev[2:5]), 3)
        sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=True, dq=dq, dk=dk, dv=dv,
                 workspace=ws, stream=stream)
        if ev is not None:
            lib.sdpa_set_timing_events(None, 0)

    # Warm up by count and by time: the clock ramps over the first ~100 ms of
    # sustained work, so at least --warmup-s seconds of steps run first.
    t_w, n_w = time.perf_counter(), 0
    while n_w < args.warmup or time.perf_counter() - t_w < args.warmup_s:
        step()
        n_w += 1
        if n_w % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup_s = time.perf_counter() - t_w
    events = [[hip.event().value for _ in range(5)] for _ in range(args.steps)]
    start, stop = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(start, sh)
    for i in range(args.steps):
        step(events[i])
    hip.record(stop, sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = hip.ms(start, stop)
    ms_step = total_ms / args.steps

    per = {"fwd": [], "bwd_dq": [], "bwd_dkdv": []}
    for ev in events:
        per["fwd"].append(hip.ms(ev[0], ev[1]))
        per["bwd_dq"].append(hip.ms(ev[2], ev[3]))     # dQ, with D = rowsum(dO * O)
        per["bwd_dkdv"].append(hip.ms(ev[3], ev[4]))
    mean = {k: statistics.fmean(v) for k, v in per.items()}
    med = {k: statistics.median(v) for k, v in per.items()}

    F = w.fwd_flops                      # counted forward flops
    step_flops = 3.5 * F                 # forward + backward (2.5x)
    value = step_flops / (ms_step / 1e3) / 1e12
    fwd_tflops = F / (med["fwd"] / 1e3) / 1e12
    bwd_ms = med["bwd_dkdv"] + med["bwd_dq"]
    bwd_tflops = 2.5 * F / (bwd_ms / 1e3) / 1e12
    # matmul flops each kernel performs per launch (per (b, h) head: s_q*s_kv*d*2 per matmul, halved causal)
    mm = F / 2.0
    kernel_flops = {"fwd": 2 * mm, "bwd_dkdv": 4 * mm, "bwd_dq": 3 * mm}
    dom = max(("fwd", "bwd_dkdv", "bwd_dq"), key=lambda k: mean[k])
    achieved = kernel_flops[dom] / (mean[dom] / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(dom), "kernel": dom,
                "kernel_ms_mean": round(mean[dom], 4)}
    log(f"[bench] per-kernel median ms: " + ", ".join(f"{k}={v:.3f}" for k, v in med.items()))
    log(f"[bench] fwd {fwd_tflops:.1f} TFLOP/s ({100 * fwd_tflops / PEAK_BF16_TFLOPS:.1f}% peak); "
        f"bwd {bwd_tflops:.1f}; fwd+bwd {value:.1f} ({100 * value / PEAK_BF16_TFLOPS:.1f}%)")

    measured = mfma_measured(sdpa, torch, hip, stream, sh)
    log(f"[bench] measured MFMA peak: {measured}")
    measured["fwd_pct_of_measured_bf16"] = round(100 * fwd_tflops / measured["bf16_tflops"], 2)
    measured["fwd_bwd_pct_of_measured_bf16"] = round(100 * value / measured["bf16_tflops"], 2)

    mods = None
    if not args.no_mods:
        # The same workload and tensors with score modifiers: ALiBi, then
        # dropout p = 0.1 (counted flops unchanged; the modifiers are VALU work).
        mods = {}
        slopes = sdpa.alibi_slopes(w.h_q, device="cuda:0")
        for name, kw in (("alibi", {"alibi_slopes": slopes}),
                         ("dropout_0.1", {"dropout_p": 0.1, "dropout_seed": 1234, "dropout_offset": 0})):
            def mstep(kw=kw):
                sdpa.fwd(g["q"], g["k"], g["v"], scale=w.scale, causal=True, out=o, lse=lse, stream=stream, **kw)
                sdpa.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, scale=w.scale, causal=True, dq=dq, dk=dk, dv=dv,
                         workspace=ws, stream=stream, **kw)
            for _ in range(args.warmup):
                mstep()
            a0, a1 = hip.event(), hip.event()
            torch.cuda.synchronize()
            hip.record(a0, sh)
            for _ in range(args.steps):
                mstep()
            hip.record(a1, sh)
            torch.cuda.synchronize()
            mms = hip.ms(a0, a1) / args.steps
            mods[name] = {"ms_per_step": round(mms, 4), "tflops": round(step_flops / (mms / 1e3) / 1e12, 2),
                          "vs_plain": round(ms_step / mms, 3)}
        log(f"[bench] score modifiers (same step): {mods}")

    fp8 = fp8_train = None
    if not args.no_fp8:
        fp8 = fp8_forward(sdpa, sdpa_inputs, torch, hip, stream, sh, args.warmup, args.steps)
        log(f"[bench] fp8 forward (b4 h8 s8192 d256, non-causal): {fp8}")
        fp8_train = fp8_hd128_forward_backward(sdpa, sdpa_inputs, torch, hip, stream, sh, args.warmup, args.steps,
                                               ms_step)
        log(f"[bench] fp8 hd128 causal forward + backward: {fp8_train}")

    dec = None
    if not args.no_decode:
        dec = decode_forward(sdpa, sdpa_inputs, torch, hip, stream, sh, args.warmup, args.steps)
        log(f"[bench] KV-cache decode: {dec}")

    vl = None
    if not args.no_varlen:
        vl = varlen_forward_backward(sdpa, sdpa_inputs, torch, hip, stream, sh, args.warmup, args.steps)
        log(f"[bench] ragged batch (padding mask): {vl}")

    cpu = None
    if args.cpu_heads > 0:
        cpu = cpu_baseline(w, ins, args.cpu_heads)
        log(f"[bench] cpu oracle: {cpu}")

    out = {
        "metric": "SDPA fwd and fwd+bwd TFLOPS and % of MFMA peak, hd128 causal bf16",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": round(warmup_s, 3),
        "warmup_steps_run": n_w,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "b": w.b, "h_q": w.h_q, "h_kv": w.h_kv, "s_q": w.s_q, "s_kv": w.s_kv,
                   "d": w.d, "causal": True, "layout": "bshd", "step": "forward + backward",
                   "parallelism": "single GPU"},
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_pct_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_bwd_tflops": round(value, 2),
        "fwd_bwd_pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "bwd_tflops": round(bwd_tflops, 2),
        "kernel_ms_median": {k: round(v, 4) for k, v in med.items()},
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "mfma_measured": measured,
        "fp8_forward": fp8,
        "fp8_hd128_forward_backward": fp8_train,
        "decode_forward": dec,
        "varlen_forward_backward": vl,
        "score_modifiers": mods,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
