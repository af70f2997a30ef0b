#!/usr/bin/env python3
"""Throughput of exact causal sliding-window attention (+ sinks) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-extras] [--no-cold] [--no-cpu-baseline] [--no-peaks]

Prints ONE JSON line.  The headline workload is the sink prefill: batch 1,
32 heads, n=32768, d=128, w=4096, g=4 sink tokens with a +4 logit offset,
bf16.  One step = one prefill launch over the whole prompt, inputs already
resident in HBM.  `value` is band-TFLOP/s: 4*d FLOP per attended (query,
key) pair (two products, a multiply-add counted as 2), pairs counted exactly
per row.

The same line carries, under "extra", every other workload, each with its
own roofline: the rolling-cache decode (batch 64, 32 heads, w=4096, g=4,
positions in [4096, 131072]; KV GB/s), its grouped-query (8 key/value heads)
and FP8-cache forms, the Mistral-shaped prefill (n=16384, w=4096), the
Gemma-3-style local prefill (16 heads, n=131072, w=1024), the Mistral-shaped
grouped-query prefill (32 query heads over 8 key/value heads), the chunked
prefill against the cache, the dilated and the landmark prefills, and the
decode step's one-token kv_append.  They run before the headline, which is
timed last.

Timing: every launch is bracketed by HIP events on the stream the kernel
runs on; `ms_per_step` is the whole timed region over K steps, `roofline`
gives the mean, median, p10 and p90 launch times.  For prefill a cold-cache
figure follows: a 1 GiB scratch write between launches evicts L2 and MALL
before each timed launch.

`roofline.traffic` is HBM bytes per launch from rocprofv3 FETCH_SIZE and
WRITE_SIZE (calibrated on a plain device copy), reported only while the
kernel sources match the ones the counters were taken on; `roofline.counters`
likewise carries the matrix-core figures of the same profiles.
`cpu_baseline` is the fp64 oracle on a bounded sample of the headline
workload, on all the host's cores and on one core.  `measured_peak` holds
what the measurement kernels of include/swa_probe.h reach on this chip (a
dense bf16 MFMA stream, a streaming HBM read); each roofline states
`frac_of_measured` beside `frac` (against the datasheet peak).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SWA prefill band-TFLOP/s and decode KV GB/s, % of MI355X peak, 1 GPU"
# The source pages' own figures, reported beside the measurement as context
# only: neither is a timing of this operation on named hardware.
CONTEXT_FROM_PAGES = {
    "flash_attention_speedup": "a factor of at most 7.6 against attention that writes its intermediates to HBM "
                               "('@akshay_pachaar: 1) Sparse Attention ...', '2. Flash Attention'; no hardware, "
                               "sizes or window given)",
    "mistral_7b_window": "w = 4096 in each of 32 layers, so information can travel about 32 x 4096 = 131072 "
                         "positions ('Sliding Window and Sparse Attention, from Longformer to CSA2', s2; the decode "
                         "workloads draw positions up to 131072)",
}
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = "sink_prefill"

PREFILL = {
    # name: (batch, heads, n, d, w, g, sink_bias, seed)
    "tiny_fp32": (1, 1, 256, 64, 64, 0, 0.0, 1),
    "mistral_prefill": (1, 32, 16384, 128, 4096, 0, 0.0, 2),
    "sink_prefill": (1, 32, 32768, 128, 4096, 4, 4.0, 3),
    "gemma3_local_prefill": (1, 16, 131072, 128, 1024, 0, 0.0, 5),
}
# grouped-query prefill: (batch, heads, kv_heads, n, d, w, g, sink_bias, seed);
# Mistral 7B's 32 query heads over 8 key/value heads
PREFILL_GQA = {
    "gqa_prefill": (1, 32, 8, 16384, 128, 4096, 0, 0.0, 9),
}
DECODE = {
    # name: (batch, heads, kv_heads, d, w, g, pos_lo, pos_hi, seed)
    "rolling_decode": (64, 32, 32, 128, 4096, 4, 4096, 131072, 4),
    # grouped-query attention: 4 query heads per key/value head
    "gqa_decode": (64, 32, 8, 128, 4096, 4, 4096, 131072, 4),
    # the rolling-cache decode over an FP8 (E4M3) cache with per-head scales
    "fp8_decode": (64, 32, 32, 128, 4096, 4, 4096, 131072, 4),
}

CHUNK = {
    # name: (batch, heads, kv_heads, t, p0, d, w, g, sink_bias, seed): a chunk of t
    # tokens at positions p0 .. p0+t-1 against a full rolling cache (Mistral 7B's
    # 32 query / 8 key-value heads and w = 4096, plus 4 sinks)
    "chunk_prefill": (1, 32, 8, 4096, 16384, 128, 4096, 4, 0.0, 6),
}

PATTERN = {
    # name: (batch, heads, n, d, kind, w, g, r, sink_bias, seed)
    # every 4th key over a 4093-position span (a 1024-key window's cost)
    "dilated_prefill": (1, 32, 16384, 128, "dilated", 1024, 0, 4, 0.0, 7),
    # Mistral's window plus 4 sinks plus landmarks every 64 positions
    "landmark_prefill": (1, 32, 16384, 128, "landmark", 4096, 4, 64, 0.0, 8),
}

# HBM traffic per launch measured with rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE per dispatch, each scaled by what the same counter reads for a
# plain device copy of known size, see --calibrate-copy), keyed by workload.
# Each entry records a digest of the kernel source it was measured on; when
# the source has changed since, the figure no longer describes the kernel and
# `traffic` is reported as null.
MEASURED_TRAFFIC = {
    "sink_prefill": {"bytes": 1074000000, "source_digest": "f47b6414d6a70bab"},
    "mistral_prefill": {"bytes": 537300000, "source_digest": "f47b6414d6a70bab"},
    "gemma3_local_prefill": {"bytes": 2253000000, "source_digest": "f47b6414d6a70bab"},
    "gqa_prefill": {"bytes": 336000000, "source_digest": "f47b6414d6a70bab"},
    "chunk_prefill": {"bytes": 122500000, "source_digest": "f47b6414d6a70bab"},
    "dilated_prefill": {"bytes": 542800000, "source_digest": "f47b6414d6a70bab"},
    "landmark_prefill": {"bytes": 553600000, "source_digest": "f47b6414d6a70bab"},
    "rolling_decode": {"bytes": 4300000000, "source_digest": "1726a2c9d6aab72a"},
    "gqa_decode": {"bytes": 1076000000, "source_digest": "1726a2c9d6aab72a"},
    "fp8_decode": {"bytes": 2151000000, "source_digest": "1726a2c9d6aab72a"},
}
# Matrix-core figures of the prefill kernels from rocprofv3 counter runs
# (SQ_INSTS_MFMA, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, SQ_BUSY_CYCLES per
# dispatch), keyed by workload, with the digest of the sources they were
# taken on (reported as null once the kernel has changed):
#   issued_per_band: MFMA FLOP issued (SQ_INSTS_MFMA x 32768) / band FLOP;
#   mfma_busy_per_simd: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs);
#   clock_ghz: GRBM_GUI_ACTIVE / 8 XCDs / kernel duration.
MEASURED_COUNTERS = {
    "sink_prefill": {"issued_per_band": 1.037, "mfma_busy_per_simd": 0.648, "clock_ghz": 1.73,
                     "valu_per_mfma": 4.71, "source_digest": "f47b6414d6a70bab"},
    "mistral_prefill": {"issued_per_band": 1.02, "mfma_busy_per_simd": 0.616, "clock_ghz": 1.77,
                        "valu_per_mfma": 4.67, "source_digest": "f47b6414d6a70bab"},
    "gemma3_local_prefill": {"issued_per_band": 1.078, "mfma_busy_per_simd": 0.484, "clock_ghz": 1.92,
                             "valu_per_mfma": 5.84, "source_digest": "f47b6414d6a70bab"},
    "gqa_prefill": {"issued_per_band": 1.02, "mfma_busy_per_simd": 0.631, "clock_ghz": 1.75,
                    "valu_per_mfma": 4.67, "source_digest": "f47b6414d6a70bab"},
    "chunk_prefill": {"issued_per_band": 1.038, "mfma_busy_per_simd": 0.57, "clock_ghz": 1.81,
                      "valu_per_mfma": 4.86, "source_digest": "f47b6414d6a70bab"},
    "dilated_prefill": {"issued_per_band": 1.08, "mfma_busy_per_simd": 0.428, "clock_ghz": 2.02,
                        "valu_per_mfma": 6.08, "source_digest": "f47b6414d6a70bab"},
    "landmark_prefill": {"issued_per_band": 1.049, "mfma_busy_per_simd": 0.592, "clock_ghz": 1.81,
                         "valu_per_mfma": 5.0, "source_digest": "f47b6414d6a70bab"},
}
CSRC = os.path.join(ROOT, "block_sparse_causal_band_amd", "csrc")


# headers each kernel source includes (the digest covers exactly what it compiles from)
KERNEL_HEADERS = {"prefill.hip": ("common.h", "schedule.h"), "decode.hip": ("common.h",)}


def kernel_source_digest(name: str) -> str:
    """Digest of the code a kernel source compiles from, comments and blank
    space left out (the kernel sources hold no string with a comment marker),
    so that an edit of a comment keeps the recorded counters."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in KERNEL_HEADERS[name] + (name,):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _measured(table, workload: str, source: str):
    entry = table.get(workload)
    if entry is None or entry["source_digest"] != kernel_source_digest(source):
        return None
    return entry


def measured_traffic(workload: str, source: str):
    entry = _measured(MEASURED_TRAFFIC, workload, source)
    return None if entry is None else entry["bytes"]


def measured_counters(workload: str):
    entry = _measured(MEASURED_COUNTERS, workload, "prefill.hip")
    return None if entry is None else {k: v for k, v in entry.items() if k != "source_digest"}


def row_pairs(i: int, w: int, g: int) -> int:
    """|A_i|: window keys min(i+1, w) plus sink keys below the window."""
    return min(i + 1, w) + min(g, max(0, i - w + 1))


def band_pairs(n: int, w: int, g: int) -> int:
    # closed form of sum_i row_pairs(i, w, g)
    m = min(n, w)
    pairs = m * (m + 1) // 2 + (n - m) * w
    if g > 0 and n > w:
        # rows i >= w see min(g, i-w+1) sinks below the window
        k = n - w  # number of rows with i - w + 1 >= 1
        full = max(0, k - g)  # rows seeing all g sinks
        ramp = k - full       # rows seeing 1..ramp sinks
        pairs += ramp * (ramp + 1) // 2 + full * g
    return pairs


def _pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    pos = (len(xs) - 1) * q
    lo = int(pos)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (pos - lo)


def _stats(per):
    return {"mean": sum(per) / len(per), "median": _pct(per, 0.5), "p10": _pct(per, 0.1), "p90": _pct(per, 0.9),
            "min": min(per), "max": max(per), "launches": len(per)}


def _events_time(fn, steps, stream, between=None):
    """Times `steps` calls of fn, each bracketed by events on `stream`.
    Returns (elapsed ms of the whole region / steps, per-call ms list).
    `between` (untimed, on the same stream) runs before each call."""
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for a, b in evs:
        if between is not None:
            between()
        a.record(stream)
        fn()
        b.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    return t0.elapsed_time(t1) / steps, per


def _run(step, steps, warmup):
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    return _events_time(step, steps, torch.cuda.current_stream())


# rates the measurement kernels reach on this chip (filled by measured_peaks)
MEASURED_PEAK = {}


def _roofline(bound, work, per, peak, unit, traffic, kernel, counters=None):
    st = _stats(per)
    achieved = work / (st["mean"] * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
    r = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
         "traffic": traffic, "kernel": kernel, "launch_ms": st,
         "frac_median": work / (st["median"] * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9) / peak,
         "counters": counters}
    if bound in MEASURED_PEAK and peak in (PEAK_BF16_TFLOPS, PEAK_HBM_GBS):
        m = MEASURED_PEAK[bound]["value"]
        r["measured_peak"] = m
        r["frac_of_measured"] = achieved / m
    return r


def measured_peaks(reps: int = 10):
    """The dense bf16 MFMA stream and the streaming HBM read of
    include/swa_probe.h, each timed with HIP events over `reps` launches
    after 3 warm-up launches; the read takes the best of a few launch shapes
    over a 4 GiB buffer.  Fills MEASURED_PEAK and returns it."""
    import torch

    import block_sparse_causal_band_amd as swa

    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()

    wg, iters = 1024, 8000
    out = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    flops = 0.0
    for _ in range(3):
        flops = swa.probe_mfma_bf16(out, wg, iters)
    _, per = _events_time(lambda: swa.probe_mfma_bf16(out, wg, iters), reps, stream)
    st = _stats(per)
    MEASURED_PEAK["mfma"] = {"value": flops / (st["median"] * 1e-3) / 1e12, "unit": "TFLOP/s",
                             "kernel": "probe_mfma_kernel (v_mfma_f32_32x32x16_bf16, register operands)",
                             "workgroups": wg, "iters": iters, "launch_ms_median": st["median"]}
    del out

    nbytes = 1 << 32
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    best = None
    for wg in (1024, 2048, 4096):
        for streams in (1, 2):
            sink = torch.zeros(wg, dtype=torch.int32, device=dev)
            for _ in range(3):
                swa.probe_hbm_read(buf, wg, streams, sink)
            _, per = _events_time(lambda: swa.probe_hbm_read(buf, wg, streams, sink), reps, stream)
            med = _stats(per)["median"]
            gbs = nbytes / (med * 1e-3) / 1e9
            if best is None or gbs > best["value"]:
                best = {"value": gbs, "unit": "GB/s", "kernel": "probe_read_kernel (16-byte non-temporal loads)",
                        "bytes": nbytes, "workgroups": wg, "streams": streams, "launch_ms_median": med}
    del buf
    torch.cuda.empty_cache()
    MEASURED_PEAK["hbm"] = best
    return MEASURED_PEAK


def bench_prefill(name, steps, warmup, cold=False):
    import torch

    import block_sparse_causal_band_amd as swa
    from block_sparse_causal_band_amd import synth

    B, H, n, d, w, g, beta, seed = PREFILL[name]
    dtype = torch.float32 if name == "tiny_fp32" else torch.bfloat16
    dev = torch.device("cuda")
    q, k, v = synth.qkv(B, H, n, d, dtype, seed=seed, device=dev)
    o = torch.empty_like(q)

    def step():
        swa.prefill(q, k, v, w=w, g=g, sink_bias=beta, out=o)

    ms_step, per = _run(step, steps, warmup)
    flops = 4.0 * d * band_pairs(n, w, g) * B * H
    peak = PEAK_BF16_TFLOPS if dtype == torch.bfloat16 else PEAK_F32_TFLOPS
    r = {
        "ms_per_step": ms_step,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "dtype": "bf16" if dtype == torch.bfloat16 else "f32",
        "config": {"workload": name, "batch": B, "heads": H, "n": n, "d": d, "w": w, "g": g,
                   "sink_bias": beta, "band_flops_per_step": flops,
                   "page_formula_flops_4nwd": 4.0 * n * w * d * B * H},
        "roofline": _roofline("mfma", flops, per, peak, "TFLOP/s", measured_traffic(name, "prefill.hip"),
                              f"prefill_bf16_kernel<{d}>" if dtype == torch.bfloat16 else f"prefill_f32_kernel<{d}>",
                              measured_counters(name)),
    }
    if cold:
        r["cold_cache"] = _cold(step, flops, peak, steps)
    del q, k, v, o
    return r


def _cold(step, flops, peak, steps):
    """Launches timed after a 1 GiB scratch write (L2 and MALL hold none of the inputs)."""
    import torch

    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    val = [0]

    def flush():
        val[0] = (val[0] + 1) & 0xFF
        scratch.fill_(val[0])

    flush()
    torch.cuda.synchronize()
    _, per = _events_time(step, min(steps, 20), torch.cuda.current_stream(), between=flush)
    st = _stats(per)
    del scratch
    return {"launch_ms": st, "value_median": flops / (st["median"] * 1e-3) / 1e12, "unit": "TFLOP/s",
            "frac_median": flops / (st["median"] * 1e-3) / 1e12 / peak,
            "note": "1 GiB scratch written before each timed launch"}


def bench_prefill_gqa(name, steps, warmup):
    import torch

    import block_sparse_causal_band_amd as swa
    from block_sparse_causal_band_amd import synth

    B, H, Hkv, n, d, w, g, beta, seed = PREFILL_GQA[name]
    dev = torch.device("cuda")
    q, k, v = synth.qkv(B, H, n, d, torch.bfloat16, seed=seed, device=dev, kv_heads=Hkv)
    o = torch.empty_like(q)

    def step():
        swa.prefill(q, k, v, w=w, g=g, sink_bias=beta, out=o)

    ms_step, per = _run(step, steps, warmup)
    flops = 4.0 * d * band_pairs(n, w, g) * B * H
    return {
        "ms_per_step": ms_step,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "dtype": "bf16",
        "config": {"workload": name, "batch": B, "heads": H, "kv_heads": Hkv, "n": n, "d": d, "w": w, "g": g,
                   "sink_bias": beta, "band_flops_per_step": flops},
        "roofline": _roofline("mfma", flops, per, PEAK_BF16_TFLOPS, "TFLOP/s", measured_traffic(name, "prefill.hip"),
                              f"prefill_bf16_kernel<{d}> (grouped query heads)", measured_counters(name)),
    }


def chunk_pairs(p0: int, t: int, w: int, g: int) -> int:
    return sum(row_pairs(p0 + i, w, g) for i in range(t))


def bench_chunk(name, steps, warmup):
    import torch

    import block_sparse_causal_band_amd as swa
    from block_sparse_causal_band_amd import synth

    B, H, Hkv, T, p0, d, w, g, beta, seed = CHUNK[name]
    dev = torch.device("cuda")
    q, kn, vn = synth.qkv(B, H, T, d, torch.bfloat16, seed=seed, device=dev, kv_heads=Hkv)
    kc = synth.normal((B, Hkv, g + w, d), seed=seed + 1, dtype=torch.bfloat16, device=dev)
    vc = synth.normal((B, Hkv, g + w, d), seed=seed + 2, dtype=torch.bfloat16, device=dev)
    pos = torch.full((B,), p0, dtype=torch.int64, device=dev)
    o = torch.empty_like(q)

    def step():
        swa.chunk_prefill(q, kn, vn, kc, vc, pos, w=w, g=g, sink_bias=beta, out=o)

    ms_step, per = _run(step, steps, warmup)
    flops = 4.0 * d * chunk_pairs(p0, T, w, g) * B * H
    return {
        "ms_per_step": ms_step,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "dtype": "bf16",
        "config": {"workload": name, "batch": B, "heads": H, "kv_heads": Hkv, "t": T, "p0": p0, "d": d, "w": w,
                   "g": g, "sink_bias": beta, "band_flops_per_step": flops},
        "roofline": _roofline("mfma", flops, per, PEAK_BF16_TFLOPS, "TFLOP/s", measured_traffic(name, "prefill.hip"),
                              f"prefill_bf16_kernel<{d},chunk>", measured_counters(name)),
    }


def pattern_pairs(n: int, kind: str, w: int, g: int, r: int) -> int:
    """Attended pairs of the fixed patterns, row by row."""
    total = 0
    for i in range(n):
        if kind == "dilated":
            total += min(w, i // r + 1)
        else:  # window + sinks, then landmarks g <= j <= i - w
            total += row_pairs(i, w, g)
            if i - w >= g:
                total += (i - w) // r - (g + r - 1) // r + 1
    return total


def bench_pattern(name, steps, warmup):
    import torch

    import block_sparse_causal_band_amd as swa
    from block_sparse_causal_band_amd import synth

    B, H, n, d, kind, w, g, r, beta, seed = PATTERN[name]
    dev = torch.device("cuda")
    q, k, v = synth.qkv(B, H, n, d, torch.bfloat16, seed=seed, device=dev)
    o = torch.empty_like(q)
    ws = torch.empty(max(swa.landmark_workspace_bytes(B, H, n, d, swa.SWA_BF16), 16), dtype=torch.uint8, device=dev)

    def step():
        if kind == "dilated":
            swa.dilated_prefill(q, k, v, w=w, r=r, out=o)
        else:
            swa.landmark_prefill(q, k, v, w=w, g=g, r=r, sink_bias=beta, out=o, workspace=ws)

    ms_step, per = _run(step, steps, warmup)
    flops = 4.0 * d * pattern_pairs(n, kind, w, g, r) * B * H
    return {
        "ms_per_step": ms_step,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "dtype": "bf16",
        "config": {"workload": name, "batch": B, "heads": H, "n": n, "d": d, "pattern": kind, "w": w, "g": g,
                   "r": r, "sink_bias": beta, "band_flops_per_step": flops},
        "roofline": _roofline("mfma", flops, per, PEAK_BF16_TFLOPS, "TFLOP/s", measured_traffic(name, "prefill.hip"),
                              ("prefill_bf16_kernel<128,strided> (dilated classes)" if kind == "dilated" else
                               "prefill_bf16_kernel<128,landmark> (landmark tiles, then window and sink tiles, one launch)"),
                              measured_counters(name)),
    }


def bench_decode(name, steps, warmup):
    import torch

    import block_sparse_causal_band_amd as swa
    from block_sparse_causal_band_amd import synth

    B, H, Hkv, d, w, g, lo, hi, seed = DECODE[name]
    dev = torch.device("cuda")
    fp8 = name.startswith("fp8")
    if fp8:
        q, kc, vc, ks, vs, pos = synth.fp8_decode_problem(B, H, Hkv, d, g + w, lo, hi, torch.bfloat16, seed=seed,
                                                          device=dev)
    else:
        q, kc, vc, pos = synth.decode_problem(B, H, d, g + w, lo, hi, torch.bfloat16, seed=seed, device=dev,
                                              kv_heads=Hkv)
    o = torch.empty_like(q)
    ws_bytes = swa.decode_workspace_bytes(B, H, d, w, g, kv_heads=Hkv)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def step():
        if fp8:
            swa.decode_fp8(q, kc, vc, ks, vs, pos, w=w, g=g, out=o, workspace=ws)
        else:
            swa.decode(q, kc, vc, pos, w=w, g=g, out=o, workspace=ws)

    ms_step, per = _run(step, steps, warmup)
    # algorithmic bytes: each (batch, key/value head)'s attended K and V rows
    # once (shared by the query heads of its group), plus q and o
    rows = sum(row_pairs(int(p), w, g) for p in pos.cpu().tolist()) * Hkv
    nbytes = rows * d * (1 if fp8 else 2) * 2 + 2 * B * H * d * 2
    r = {
        "ms_per_step": ms_step,
        "value": nbytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "dtype": "fp8_e4m3 cache, bf16 q/o, fp32 arithmetic" if fp8 else "bf16",
        "config": {"workload": name, "batch": B, "heads": H, "kv_heads": Hkv, "d": d, "w": w, "g": g,
                   "positions": [lo, hi], "kv_bytes_per_step": nbytes},
        "roofline": _roofline("hbm", nbytes, per, PEAK_HBM_GBS, "GB/s", measured_traffic(name, "decode.hip"),
                              ("decode_kernel<bf16,fp8x16,128>" if fp8 else
                               "decode_mfma_kernel<128>" if Hkv < H else "decode_kernel<bf16,bf16,128>")),
    }
    del q, kc, vc, o
    return r


def bench_kv_append(name, steps, warmup):
    """The decode step's append: one new token per (batch, key/value head)
    written to its ring row (and sink row below g)."""
    import torch

    import block_sparse_causal_band_amd as swa
    from block_sparse_causal_band_amd import synth

    B, H, Hkv, d, w, g, lo, hi, seed = DECODE[name]
    dev = torch.device("cuda")
    _, kc, vc, pos = synth.decode_problem(B, H, d, g + w, lo, hi, torch.bfloat16, seed=seed, device=dev,
                                          kv_heads=Hkv)
    kn = synth.normal((B, Hkv, 1, d), seed=seed + 7, dtype=torch.bfloat16, device=dev)
    vn = synth.normal((B, Hkv, 1, d), seed=seed + 8, dtype=torch.bfloat16, device=dev)

    def step():
        swa.kv_append(kc, vc, kn, vn, pos, w=w, g=g)

    ms_step, per = _run(step, steps, warmup)
    writes = sum(2 if int(p) < g else 1 for p in pos.cpu().tolist()) * Hkv
    nbytes = 2 * B * Hkv * d * 2 + writes * 2 * d * 2  # k_new, v_new read; cache rows written
    return {"ms_per_step": ms_step, "value": nbytes / (ms_step * 1e-3) / 1e9, "unit": "GB/s", "dtype": "bf16",
            "config": {"workload": f"{name} append (1 token)", "batch": B, "kv_heads": Hkv, "d": d, "w": w, "g": g,
                       "bytes_per_step": nbytes},
            "roofline": _roofline("hbm", nbytes, per, PEAK_HBM_GBS, "GB/s", None, "kv_append_kernel<bf16>")}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_prefill(name, budget_s=12.0, single_s=3.0):
    """The fp64 oracle, as it stands, on whole heads of the same workload until
    about budget_s seconds of CPU work on every core, then on one core for
    about single_s seconds; rates in band-TFLOP/s."""
    import numpy as np
    import torch

    import oracle
    from block_sparse_causal_band_amd import synth

    B, H, n, d, w, g, beta, seed = PREFILL[name]
    dtype = torch.float32 if name == "tiny_fp32" else torch.bfloat16
    q, k, v = synth.qkv(B, H, n, d, dtype, seed=seed, device="cpu")
    orc = oracle.default()
    threads = orc.num_threads()
    rows_per_chunk = 512 if n >= 4096 else n

    def run(budget, nthreads, chunk):
        done_pairs = done_rows = heads = 0
        t0 = time.perf_counter()
        # whole heads, each from its last rows backwards (full-window rows are
        # the bulk of the workload), until the budget is spent
        for bh in range(B * H):
            if time.perf_counter() - t0 >= budget:
                break
            b, h = divmod(bh, H)
            heads += 1
            start = n - chunk
            while time.perf_counter() - t0 < budget and start > -chunk:
                rows = np.arange(max(0, start), start + chunk)
                orc.prefill(q[b, h], k[b, h], v[b, h], w=w, g=g, beta=beta, rows=rows, nthreads=nthreads)
                done_pairs += sum(row_pairs(int(i), w, g) for i in rows)
                done_rows += len(rows)
                start -= chunk
        return done_pairs, done_rows, heads, time.perf_counter() - t0

    pairs, rows, heads, dt = run(budget_s, threads, rows_per_chunk)
    pairs1, rows1, _, dt1 = run(single_s, 1, rows_per_chunk)
    return {
        "value": 4.0 * d * pairs / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{rows} query rows over {heads} head(s) of {name} (each head from its last row backwards), "
                  f"fp64, {dt:.1f} s on {threads} threads",
        "nproc": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "cpu_model": _cpu_model(),
        "per_core": {"value": 4.0 * d * pairs1 / dt1 / 1e12, "unit": "TFLOP/s",
                     "sample": f"{rows1} rows of the first head from its last row backwards, 1 thread, {dt1:.1f} s"},
        "full_workload_s_estimate": 4.0 * d * band_pairs(n, w, g) * B * H / (4.0 * d * pairs / dt),
    }


def cpu_baseline_decode(name, budget_s=10.0):
    import numpy as np
    import torch

    import oracle
    from block_sparse_causal_band_amd import synth

    B, H, Hkv, d, w, g, lo, hi, seed = DECODE[name]
    orc = oracle.default()
    rng = np.random.default_rng(seed)
    nk = g + w
    units = 64
    q = synth.normal((units, d), seed=seed, dtype=torch.bfloat16)
    kk = synth.normal((units, nk, d), seed=seed + 2, dtype=torch.bfloat16)
    vv = synth.normal((units, nk, d), seed=seed + 3, dtype=torch.bfloat16)
    done_bytes = 0
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        ps = rng.integers(lo, hi + 1, units)
        kpos = np.stack([np.concatenate([np.arange(p - w + 1, p + 1), np.arange(0, min(g, p - w + 1))])
                         for p in ps])
        orc.decode(q, ps, kpos, kk, vv, w=w, g=g)
        eb = 1 if name.startswith("fp8") else 2  # cache bytes per element
        done_bytes += sum(row_pairs(int(p), w, g) for p in ps) * d * eb * 2 + 2 * units * d * 2
        done += units
    dt = time.perf_counter() - t0
    return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{done} (batch, head) queries of {name}, fp64, {dt:.1f} s", "nproc": os.cpu_count(),
            "cpu_model": _cpu_model()}


def calibrate_copy(steps: int, nbytes: int = 1 << 30):
    """A plain device-to-device copy of known size, for scaling the HBM
    byte counters: FETCH_SIZE and WRITE_SIZE of these dispatches should each
    read nbytes."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes,
                      "copies": steps, "ms_per_copy": dt * 1e3, "GB_per_s_read_plus_write": 2 * nbytes / dt / 1e9}),
          flush=True)


def _bench(name, steps, warmup, cold=False):
    if name in PREFILL:
        return bench_prefill(name, steps, warmup, cold=cold)
    if name in PREFILL_GQA:
        return bench_prefill_gqa(name, steps, warmup)
    if name in CHUNK:
        return bench_chunk(name, steps, warmup)
    if name in PATTERN:
        return bench_pattern(name, steps, warmup)
    return bench_decode(name, steps, warmup)


# untimed launches before each extra workload (the headline takes --warmup)
EXTRA_WARMUP = 40


def _brief(r):
    keep = ("value", "unit", "ms_per_step", "dtype", "config", "roofline", "cold_cache")
    return {k: r[k] for k in keep if k in r}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    names = sorted(PREFILL) + sorted(PREFILL_GQA) + sorted(DECODE) + sorted(CHUNK) + sorted(PATTERN)
    ap.add_argument("--workload", default=HEADLINE, choices=names)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="time only the selected workload")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache prefill figure")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA and HBM peaks")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(heads and batch would shard with no exchange between GPUs). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.steps)
        return

    if not args.no_peaks:
        measured_peaks()
    extra = {}
    if not args.no_extras and args.workload == HEADLINE:
        # the other workloads first: the headline is timed last, on a chip
        # whose clock has settled under load
        # (each with at least EXTRA_WARMUP untimed launches: with fewer, the
        # clock has not settled on the short decode kernels)
        wu = max(args.warmup, EXTRA_WARMUP)
        for name in ("rolling_decode", "gqa_decode", "fp8_decode", "mistral_prefill", "gemma3_local_prefill",
                     "gqa_prefill", "chunk_prefill", "dilated_prefill", "landmark_prefill"):
            extra[name] = dict(_brief(_bench(name, args.steps, wu)), warmup=wu)
            torch.cuda.empty_cache()
        extra["kv_append"] = dict(_brief(bench_kv_append("rolling_decode", args.steps, wu)), warmup=wu)
        torch.cuda.empty_cache()
    r = _bench(args.workload, args.steps, args.warmup,
               cold=(not args.no_cold and args.workload in PREFILL))
    line = {
        "metric": METRIC,
        "value": r["value"],
        "unit": r["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic: iid N(0,1) inputs from seeded torch generators, rounded to the dtype",
        "config": r["config"],
        "roofline": r["roofline"],
    }
    line["roofline"]["frac_str"] = f"{100 * r['roofline']['frac']:.1f}% of MI355X peak"
    if MEASURED_PEAK:
        line["measured_peak"] = MEASURED_PEAK
    if "cold_cache" in r:
        line["cold_cache"] = r["cold_cache"]
    if extra:
        line["extra"] = extra
    line["context_from_pages"] = CONTEXT_FROM_PAGES
    if not args.no_cpu_baseline:
        if args.workload in PREFILL:
            line["cpu_baseline"] = cpu_baseline_prefill(args.workload)
        elif args.workload in DECODE:
            line["cpu_baseline"] = cpu_baseline_decode(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
