"""Dilated windows and landmarks on the HIP path (through the C ABI) against
the oracle's pattern rows (oracle/patterns.py): fp32 1e-4, bf16 2e-2 max-abs,
outputs and LSE.  A dilation of 1 must equal the plain prefill bit for bit
(the same tiles and arithmetic)."""
import numpy as np
import pytest
import torch

import block_sparse_causal_band_amd as swa
import oracle
from block_sparse_causal_band_amd import synth
from oracle import patterns

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda")


def _tol(dtype):
    return 2e-2 if dtype == torch.bfloat16 else 1e-4


def _check(q, k, v, o, lse, kind, w, g, r, beta, rows=None):
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    tol = _tol(q.dtype)
    for b in range(B):
        for h in range(H):
            j = oracle.kv_head_of(h, H, Hkv)
            ro, rl = patterns.prefill(q[b, h].double().cpu().numpy(), k[b, j].double().cpu().numpy(),
                                      v[b, j].double().cpu().numpy(), kind, w=w, g=g, r=r, beta=beta, rows=rows)
            go = o[b, h].float().cpu().numpy()
            gl = lse[b, h].cpu().numpy()
            if rows is not None:
                go, gl = go[rows], gl[rows]
            assert np.all(np.isfinite(go))
            err = float(np.max(np.abs(go - ro)))
            assert err <= tol, f"{kind} b{b} h{h}: max-abs {err:.3g}"
            assert float(np.max(np.abs(gl - rl))) <= tol


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n,w,r", [(300, 16, 4), (517, 70, 3), (200, 5, 64), (130, 200, 2), (64, 1, 5)])
def test_dilated_vs_oracle(dtype, d, n, w, r):
    dev = _dev()
    q, k, v = synth.qkv(2, 2, n, d, dtype, seed=91, device=dev)
    o, lse = swa.dilated_prefill(q, k, v, w=w, r=r, return_lse=True)
    torch.cuda.synchronize()
    _check(q, k, v, o, lse, "dilated", w, 0, r, 0.0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dilation_one_is_plain_prefill(dtype):
    dev = _dev()
    q, k, v = synth.qkv(1, 4, 1000, 128, dtype, seed=92, device=dev)
    a, la = swa.dilated_prefill(q, k, v, w=300, r=1, return_lse=True)
    b, lb = swa.prefill(q, k, v, w=300, g=0, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n,w,g,r,beta", [(300, 16, 0, 4, 0.0), (517, 64, 4, 32, 2.0), (400, 100, 1, 7, -1.0),
                                          (260, 8, 0, 1, 0.0), (150, 20, 3, 500, 0.5)])
def test_landmark_vs_oracle(dtype, d, n, w, g, r, beta):
    dev = _dev()
    q, k, v = synth.qkv(2, 2, n, d, dtype, seed=93, device=dev)
    o, lse = swa.landmark_prefill(q, k, v, w=w, g=g, r=r, sink_bias=beta, return_lse=True)
    torch.cuda.synchronize()
    _check(q, k, v, o, lse, "landmark", w, g, r, beta)


@pytest.mark.parametrize("d", [64, 128])
def test_landmark_without_lse_output(d):
    """Without an LSE output the window part's LSE goes to the workspace; o is
    the same bit for bit."""
    dev = _dev()
    q, k, v = synth.qkv(2, 2, 517, d, torch.bfloat16, seed=95, device=dev)
    a, _ = swa.landmark_prefill(q, k, v, w=64, g=4, r=32, sink_bias=2.0, return_lse=True)
    b = swa.landmark_prefill(q, k, v, w=64, g=4, r=32, sink_bias=2.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("kind", ["dilated", "landmark"])
def test_patterns_gqa(kind):
    dev = _dev()
    H, Hkv, n, w, r = 8, 2, 333, 40, 4
    q, k, v = synth.qkv(1, H, n, 128, torch.bfloat16, seed=94, device=dev, kv_heads=Hkv)
    if kind == "dilated":
        o, lse = swa.dilated_prefill(q, k, v, w=w, r=r, return_lse=True)
    else:
        o, lse = swa.landmark_prefill(q, k, v, w=w, g=2, r=r, sink_bias=1.0, return_lse=True)
    torch.cuda.synchronize()
    _check(q, k, v, o, lse, kind, w, 0 if kind == "dilated" else 2, r, 0.0 if kind == "dilated" else 1.0)


@pytest.mark.parametrize("kind", ["dilated", "landmark"])
def test_patterns_full_size_sampled(kind):
    """Mistral-shaped rows (batch 1, 32 heads, n=16384, d=128): a dilated
    window of 1024 every 4th key, and a 4096 window with 4 sinks and
    landmarks every 64; 64 sampled rows of 4 heads against the oracle."""
    dev = _dev()
    n = 16384
    q, k, v = synth.qkv(1, 32, n, 128, torch.bfloat16, seed=95, device=dev)
    if kind == "dilated":
        w, g, r, beta = 1024, 0, 4, 0.0
        o, lse = swa.dilated_prefill(q, k, v, w=w, r=r, return_lse=True)
    else:
        w, g, r, beta = 4096, 4, 64, 0.0
        o, lse = swa.landmark_prefill(q, k, v, w=w, g=g, r=r, return_lse=True)
    torch.cuda.synchronize()
    rows = sorted(set(np.random.default_rng(95).integers(0, n, 64).tolist()) | {0, n - 1})
    _check(q[:, :4], k[:, :4], v[:, :4], o[:, :4], lse[:, :4], kind, w, g, r, beta, rows=rows)
