"""Seeded synthetic inputs.

Shared by the tests, the smoke check and the benchmark.  This module draws
random numbers and nothing else: it holds none of the attention arithmetic
(no masks, no cache-slot arithmetic, no softmax), so the HIP path and the
oracle can both take their inputs from it without sharing any of the method.

Recipe (the same for every caller):
  * Q, K, V of one prefill problem are fp32 standard normals drawn from one
    ``torch.Generator`` seeded with ``seed``, in the order Q, K, V, then
    rounded (round-to-nearest-even) to the requested dtype;
  * a decode problem draws its query [B, H, d], then the K cache and V cache
    [B, H, rows, d], all N(0, 1), in that order, then the query positions
    uniform over [lo, hi] (int64) from a second generator seeded ``seed + 1``.
"""
from __future__ import annotations

import torch


def _gen(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed: int, dtype=torch.float32, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=device).to(dtype)


def qkv(batch: int, heads: int, n: int, d: int, dtype, seed: int, device="cpu", kv_heads: int | None = None):
    """Q [batch, heads, n, d] and K, V [batch, kv_heads (default heads), n, d],
    iid N(0, 1), rounded to dtype."""
    g = _gen(seed, device)
    out = []
    for i in range(3):
        hh = heads if (i == 0 or kv_heads is None) else kv_heads
        out.append(torch.randn(batch, hh, n, d, generator=g, dtype=torch.float32, device=device).to(dtype))
    return tuple(out)


def decode_problem(batch: int, heads: int, d: int, rows: int, lo: int, hi: int, dtype,
                   seed: int, device="cpu", kv_heads: int | None = None):
    """(q [B,H,d], k_cache [B,Hkv,rows,d], v_cache [B,Hkv,rows,d], pos [B] int64
    in [lo, hi]); Hkv = kv_heads, default H."""
    g = _gen(seed, device)
    hk = heads if kv_heads is None else kv_heads
    q = torch.randn(batch, heads, d, generator=g, dtype=torch.float32, device=device).to(dtype)
    kc = torch.randn(batch, hk, rows, d, generator=g, dtype=torch.float32, device=device).to(dtype)
    vc = torch.randn(batch, hk, rows, d, generator=g, dtype=torch.float32, device=device).to(dtype)
    gp = _gen(seed + 1, "cpu")
    pos = torch.randint(lo, hi + 1, (batch,), generator=gp, dtype=torch.int64).to(device)
    return q, kc, vc, pos


def fp8_decode_problem(batch: int, heads: int, kv_heads: int, d: int, rows: int, lo: int, hi: int, q_dtype,
                       seed: int, device="cpu"):
    """(q [B,H,d], k_cache, v_cache [B,Hkv,rows,d] uint8, k_scale, v_scale [B,Hkv] fp32,
    pos [B] int64 in [lo, hi]): cache bytes are torch's float8_e4m3fn casts of
    N(0, 1) draws (so no NaN code appears), scales uniform in [0.25, 2]."""
    g = _gen(seed, device)
    q = torch.randn(batch, heads, d, generator=g, dtype=torch.float32, device=device).to(q_dtype)
    kc = torch.randn(batch, kv_heads, rows, d, generator=g, dtype=torch.float32, device=device)
    kc = kc.to(torch.float8_e4m3fn).view(torch.uint8)
    vc = torch.randn(batch, kv_heads, rows, d, generator=g, dtype=torch.float32, device=device)
    vc = vc.to(torch.float8_e4m3fn).view(torch.uint8)
    ks = torch.rand(batch, kv_heads, generator=g, dtype=torch.float32, device=device) * 1.75 + 0.25
    vs = torch.rand(batch, kv_heads, generator=g, dtype=torch.float32, device=device) * 1.75 + 0.25
    gp = _gen(seed + 1, "cpu")
    pos = torch.randint(lo, hi + 1, (batch,), generator=gp, dtype=torch.int64).to(device)
    return q, kc, vc, ks, vs, pos
