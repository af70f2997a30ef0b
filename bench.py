#!/usr/bin/env python3
"""Throughput of exact causal sliding-window attention (+ sinks) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints ONE JSON line.  The default workload is the Mistral-7B-shaped prefill
(batch 1, 32 heads, n=16384, d=128, w=4096, bf16): one step = one prefill
launch over the whole prompt, inputs already resident in HBM.  `value` is
band-TFLOP/s: 4*d FLOP per attended (query, key) pair (two products, a
multiply-add counted as 2), attended pairs counted exactly per row.  The
same line carries the rolling-cache decode workload (batch 64, 32 heads,
d=128, w=4096, g=4, positions in [4096, 131072]) as KV GB/s: bytes of the
key/value rows each query attends, plus q and o.

`roofline` is for the dominant kernel of the line's workload, timed with
events on the stream the kernel runs on.  `cpu_baseline` is the fp64 oracle
on a bounded sample of the same workload, on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SWA prefill band-TFLOP/s and decode KV GB/s, % of MI355X peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

PREFILL = {
    # name: (batch, heads, n, d, w, g, sink_bias, seed)
    "tiny_fp32": (1, 1, 256, 64, 64, 0, 0.0, 1),
    "mistral_prefill": (1, 32, 16384, 128, 4096, 0, 0.0, 2),
    "sink_prefill": (1, 32, 32768, 128, 4096, 4, 4.0, 3),
    "gemma3_local_prefill": (1, 16, 131072, 128, 1024, 0, 0.0, 5),
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
    "mistral_prefill": {"bytes": 537654927, "source_digest": "f4050d4cfde5a500"},
    "sink_prefill": {"bytes": 1074220565, "source_digest": "f4050d4cfde5a500"},
    "gemma3_local_prefill": {"bytes": 2226296863, "source_digest": "f4050d4cfde5a500"},
    "chunk_prefill": {"bytes": 140024216, "source_digest": "f4050d4cfde5a500"},
    "rolling_decode": {"bytes": 4300265431, "source_digest": "1197048432c9c06b"},
    "gqa_decode": {"bytes": 1076057369, "source_digest": "1197048432c9c06b"},
    "fp8_decode": {"bytes": 2151013950, "source_digest": "1197048432c9c06b"},
}
CSRC = os.path.join(ROOT, "block_sparse_causal_band_amd", "csrc")


# headers each kernel source includes (the digest covers exactly what it compiles from)
KERNEL_HEADERS = {"prefill.hip": ("common.h", "schedule.h"), "decode.hip": ("common.h",)}


def kernel_source_digest(name: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_HEADERS[name] + (name,):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, source: str):
    entry = MEASURED_TRAFFIC.get(workload)
    if entry is None or entry["source_digest"] != kernel_source_digest(source):
        return None
    return entry["bytes"]


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


def _events_time(fn, steps, stream):
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    total = t0.elapsed_time(t1)
    return total / steps, sum(per) / len(per), per


def bench_prefill(name, steps, warmup):
    import torch

    import block_sparse_causal_band_amd as swa
    from block_sparse_causal_band_amd import synth

    B, H, n, d, w, g, beta, seed = PREFILL[name]
    dtype = torch.float32 if name == "tiny_fp32" else torch.bfloat16
    dev = torch.device("cuda")
    q, k, v = synth.qkv(B, H, n, d, dtype, seed=seed, device=dev)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step():
        swa.prefill(q, k, v, w=w, g=g, sink_bias=beta, out=o)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms_step, ms_launch, per = _events_time(step, steps, stream)
    flops = 4.0 * d * band_pairs(n, w, g) * B * H
    peak = PEAK_BF16_TFLOPS if dtype == torch.bfloat16 else PEAK_F32_TFLOPS
    achieved = flops / (ms_launch * 1e-3) / 1e12
    traffic = measured_traffic(name, "prefill.hip")
    return {
        "ms_per_step": ms_step,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "dtype": "bf16" if dtype == torch.bfloat16 else "f32",
        "config": {"workload": name, "batch": B, "heads": H, "n": n, "d": d, "w": w, "g": g,
                   "sink_bias": beta, "band_flops_per_step": flops,
                   "page_formula_flops_4nwd": 4.0 * n * w * d * B * H},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": f"prefill_bf16_kernel<{d},4>" if dtype == torch.bfloat16 else f"prefill_f32_kernel<{d}>",
                     "avg_launch_ms": ms_launch, "min_launch_ms": min(per)},
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
    stream = torch.cuda.current_stream()

    def step():
        swa.chunk_prefill(q, kn, vn, kc, vc, pos, w=w, g=g, sink_bias=beta, out=o)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms_step, ms_launch, per = _events_time(step, steps, stream)
    flops = 4.0 * d * chunk_pairs(p0, T, w, g) * B * H
    achieved = flops / (ms_launch * 1e-3) / 1e12
    return {
        "ms_per_step": ms_step,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "dtype": "bf16",
        "config": {"workload": name, "batch": B, "heads": H, "kv_heads": Hkv, "t": T, "p0": p0, "d": d, "w": w,
                   "g": g, "sink_bias": beta, "band_flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(name, "prefill.hip"),
                     "kernel": f"prefill_bf16_kernel<{d},4,chunk>",
                     "avg_launch_ms": ms_launch, "min_launch_ms": min(per)},
    }


def cpu_baseline_chunk(name, budget_s=12.0):
    """The fp64 oracle on chunk rows of the same workload (each row given the
    window and sink rows it attends), until about budget_s seconds."""
    import numpy as np
    import torch

    import oracle
    from block_sparse_causal_band_amd import synth

    B, H, Hkv, T, p0, d, w, g, beta, seed = CHUNK[name]
    orc = oracle.default()
    units = 32
    nk = w + g
    q = synth.normal((units, d), seed=seed, dtype=torch.bfloat16)
    kk = synth.normal((units, nk, d), seed=seed + 1, dtype=torch.bfloat16)
    vv = synth.normal((units, nk, d), seed=seed + 2, dtype=torch.bfloat16)
    rng = np.random.default_rng(seed)
    done_pairs, done = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        ps = p0 + rng.integers(0, T, units)
        kpos = np.stack([np.concatenate([np.arange(p - w + 1, p + 1), np.arange(0, min(g, p - w + 1))]) for p in ps])
        orc.decode(q, ps, kpos, kk, vv, w=w, g=g, beta=beta)
        done_pairs += sum(row_pairs(int(p), w, g) for p in ps)
        done += units
    dt = time.perf_counter() - t0
    return {"value": 4.0 * d * done_pairs / dt / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(),
            "kind": "oracle", "sample": f"{done} chunk rows of {name} (random rows, each with its {nk} attended keys), "
                                        f"fp64, {dt:.1f} s"}


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
    stream = torch.cuda.current_stream()

    def step():
        if kind == "dilated":
            swa.dilated_prefill(q, k, v, w=w, r=r, out=o)
        else:
            swa.landmark_prefill(q, k, v, w=w, g=g, r=r, sink_bias=beta, out=o, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms_step, ms_launch, per = _events_time(step, steps, stream)
    flops = 4.0 * d * pattern_pairs(n, kind, w, g, r) * B * H
    achieved = flops / (ms_launch * 1e-3) / 1e12
    return {
        "ms_per_step": ms_step,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "dtype": "bf16",
        "config": {"workload": name, "batch": B, "heads": H, "n": n, "d": d, "pattern": kind, "w": w, "g": g,
                   "r": r, "sink_bias": beta, "band_flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": ("prefill_bf16_kernel<128,4,strided> (dilated classes)" if kind == "dilated" else
                                "window prefill + landmark part merged in its epilogue (one call)"),
                     "avg_launch_ms": ms_launch, "min_launch_ms": min(per)},
    }


def cpu_baseline_pattern(name, budget_s=12.0):
    """The oracle's pattern rows (oracle/patterns.py, fp64 numpy) on the last
    rows of one head of the same workload, until about budget_s seconds."""
    import numpy as np
    import torch

    from block_sparse_causal_band_amd import synth
    from oracle import patterns

    B, H, n, d, kind, w, g, r, beta, seed = PATTERN[name]
    q, k, v = synth.qkv(1, 1, n, d, torch.bfloat16, seed=seed, device="cpu")
    qh, kh, vh = (t[0, 0].double().numpy() for t in (q, k, v))
    done_pairs, done, t0 = 0, 0, time.perf_counter()
    i = n - 1
    while time.perf_counter() - t0 < budget_s and i >= 0:
        rows = np.arange(max(0, i - 63), i + 1)
        patterns.prefill(qh, kh, vh, kind, w=w, g=g, r=r, beta=beta, rows=rows)
        for j in rows:
            done_pairs += len(patterns.read_set(int(j), kind, w, g, r))
        done += len(rows)
        i -= 64
    dt = time.perf_counter() - t0
    return {"value": 4.0 * d * done_pairs / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} rows of one head of {name} (from the last row back), fp64 numpy, {dt:.1f} s"}


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
    stream = torch.cuda.current_stream()

    def step():
        if fp8:
            swa.decode_fp8(q, kc, vc, ks, vs, pos, w=w, g=g, out=o, workspace=ws)
        else:
            swa.decode(q, kc, vc, pos, w=w, g=g, out=o, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms_step, ms_launch, per = _events_time(step, steps, stream)
    # algorithmic bytes: each (batch, key/value head)'s attended K and V rows
    # once (shared by the query heads of its group), plus q and o
    rows = sum(row_pairs(int(p), w, g) for p in pos.cpu().tolist()) * Hkv
    nbytes = rows * d * (1 if fp8 else 2) * 2 + 2 * B * H * d * 2
    achieved = nbytes / (ms_launch * 1e-3) / 1e9
    traffic = measured_traffic(name, "decode.hip")
    return {
        "ms_per_step": ms_step,
        "value": nbytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "dtype": "bf16",
        "config": {"workload": name, "batch": B, "heads": H, "kv_heads": Hkv, "d": d, "w": w, "g": g,
                   "positions": [lo, hi], "kv_bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": ("decode_kernel<bf16,fp8x16,128>" if fp8 else
                                "decode_mfma_kernel<128>" if Hkv < H else "decode_kernel<bf16,bf16,128>"),
                     "avg_launch_ms": ms_launch, "min_launch_ms": min(per)},
    }


def cpu_baseline_prefill(name, budget_s=12.0):
    """The fp64 oracle, as it stands, on whole heads of the same workload until
    about budget_s seconds of CPU work; rate in band-TFLOP/s."""
    import numpy as np
    import torch

    import oracle
    from block_sparse_causal_band_amd import synth

    B, H, n, d, w, g, beta, seed = PREFILL[name]
    dtype = torch.float32 if name == "tiny_fp32" else torch.bfloat16
    q, k, v = synth.qkv(B, H, n, d, dtype, seed=seed, device="cpu")
    orc = oracle.default()
    rows_per_chunk = 512 if n >= 4096 else n
    done_pairs = 0
    done_rows = 0
    heads_touched = 0
    t0 = time.perf_counter()
    # whole heads, each from its last rows backwards (full-window rows are the
    # bulk of the workload), until the budget is spent
    for bh in range(B * H):
        if time.perf_counter() - t0 >= budget_s:
            break
        b, h = divmod(bh, H)
        heads_touched += 1
        start = n - rows_per_chunk
        while time.perf_counter() - t0 < budget_s and start > -rows_per_chunk:
            rows = np.arange(max(0, start), start + rows_per_chunk)
            orc.prefill(q[b, h], k[b, h], v[b, h], w=w, g=g, beta=beta, rows=rows)
            done_pairs += sum(row_pairs(int(i), w, g) for i in rows)
            done_rows += len(rows)
            start -= rows_per_chunk
    dt = time.perf_counter() - t0
    return {
        "value": 4.0 * d * done_pairs / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "sample": f"{done_rows} query rows over {heads_touched} head(s) of {name} (each head from its "
                  f"last row backwards), fp64, {dt:.1f} s",
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
            "sample": f"{done} (batch, head) queries of {name}, fp64, {dt:.1f} s"}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clock settles over the first ~25 launches of a busy kernel (power
    # management); the default warmup keeps the timed launches past that
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="mistral_prefill", choices=sorted(PREFILL) + sorted(DECODE) + sorted(CHUNK) + sorted(PATTERN))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode figures on a prefill line")
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

    if args.workload in PREFILL:
        r = bench_prefill(args.workload, args.steps, args.warmup)
    elif args.workload in CHUNK:
        r = bench_chunk(args.workload, args.steps, args.warmup)
    elif args.workload in PATTERN:
        r = bench_pattern(args.workload, args.steps, args.warmup)
    else:
        r = bench_decode(args.workload, args.steps, args.warmup)
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
    if args.workload in PREFILL and not args.no_decode:
        dname = "rolling_decode"
        dr = bench_decode(dname, args.steps, args.warmup)
        line["decode"] = {"value": dr["value"], "unit": dr["unit"], "ms_per_step": dr["ms_per_step"],
                          "config": dr["config"], "roofline": dr["roofline"]}
    if not args.no_cpu_baseline:
        if args.workload in PREFILL:
            line["cpu_baseline"] = cpu_baseline_prefill(args.workload)
        elif args.workload in CHUNK:
            line["cpu_baseline"] = cpu_baseline_chunk(args.workload)
        elif args.workload in PATTERN:
            line["cpu_baseline"] = cpu_baseline_pattern(args.workload)
        else:
            line["cpu_baseline"] = cpu_baseline_decode(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
