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
from tests.parity import gate

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
            gate(go, ro, q.dtype, f"{kind} b{b} h{h}", tol=tol)
            gate(gl, rl, q.dtype, f"{kind} lse", tol=tol)


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
def test_patterns_random_shapes(dtype):
    """Seeded random dilated and landmark shapes: ragged n, windows below and
    above a key tile, strides from 1 to past the sequence, sinks, grouped
    heads and both head sizes; every row against the oracle."""
    dev = _dev()
    rng = np.random.default_rng(4242)
    for case in range(8):
        kind = "dilated" if case % 2 == 0 else "landmark"
        n = int(rng.integers(1, 900))
        w = int(rng.integers(1, 300))
        r = int(rng.choice([1, 2, 3, 5, 16, 64, 1000]))
        g = 0 if kind == "dilated" else int(rng.choice([0, 1, 4, 70]))
        beta = 0.0 if kind == "dilated" else float(rng.uniform(-2.0, 4.0))
        d = int(rng.choice([64, 128]))
        H, Hkv = [(2, 2), (4, 2), (3, 1), (2, 1)][case % 4]
        print(f"case {case}: {kind} n={n} w={w} r={r} g={g} d={d} H={H}/{Hkv} {dtype}", flush=True)
        q, k, v = synth.qkv(1, H, n, d, dtype, seed=500 + case, device=dev, kv_heads=Hkv)
        if kind == "dilated":
            o, lse = swa.dilated_prefill(q, k, v, w=w, r=r, return_lse=True)
        else:
            o, lse = swa.landmark_prefill(q, k, v, w=w, g=g, r=r, sink_bias=beta, return_lse=True)
        torch.cuda.synchronize()
        _check(q, k, v, o, lse, kind, w, g, r, beta)


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
@pytest.mark.parametrize("n,w,g,r,beta", [
    (2000, 64, 10, 4, 1.0),   # 484 landmarks: eight landmark tiles per late block, sinks past one stride
    (1000, 50, 0, 1, 0.0),    # every position a landmark: full causal attention
    (777, 130, 5, 5, 1.5),    # sinks end on a landmark; ragged n
    (1300, 200, 64, 3, -2.0), # 64 sinks: the landmark range starts inside the second tile
    (4200, 4096, 4, 64, 4.0), # the window of the Mistral-shaped workload: one short landmark tile
])
def test_landmark_tiles_vs_oracle(d, n, w, g, r, beta):
    """bf16 runs every landmark tile of a query block (K/V rows strided by r)
    and then its window and sink tiles through one online softmax: many
    landmark tiles, none, a range starting past tile 0, full causal."""
    dev = _dev()
    q, k, v = synth.qkv(1, 2, n, d, torch.bfloat16, seed=96, device=dev)
    print(f"landmark bf16 d={d} n={n} w={w} g={g} r={r}", flush=True)
    o, lse = swa.landmark_prefill(q, k, v, w=w, g=g, r=r, sink_bias=beta, return_lse=True)
    torch.cuda.synchronize()
    rows = None if n <= 1000 else sorted(set(range(0, n, 7)) | set(range(n - 130, n)))
    _check(q, k, v, o, lse, "landmark", w, g, r, beta, rows=rows)


def test_landmark_every_position_is_causal_attention():
    """r = 1 makes every position below the window a landmark: the union is
    plain causal attention (prefill with w >= n), up to rounding order."""
    dev = _dev()
    q, k, v = synth.qkv(1, 4, 700, 128, torch.bfloat16, seed=97, device=dev)
    a, la = swa.landmark_prefill(q, k, v, w=40, g=0, r=1, return_lse=True)
    b, lb = swa.prefill(q, k, v, w=700, g=0, return_lse=True)
    torch.cuda.synchronize()
    gate(a.float().cpu().numpy(), b.float().cpu().numpy(), torch.bfloat16, "landmark r=1 vs causal")
    gate(la.cpu().numpy(), lb.cpu().numpy(), torch.bfloat16, "landmark r=1 vs causal lse")


@pytest.mark.parametrize("d", [64, 128])
def test_landmark_without_lse_output(d):
    """o is the same bit for bit with and without an LSE output."""
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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("kind", ["dilated", "landmark"])
def test_huge_stride_equals_stride_n(dtype, kind):
    """Any stride r >= n reads the same keys as r = n (dilated: each query only
    itself; landmarks: position 0 only), so a stride far past n -- whose row
    offsets would overflow 32 bits -- gives the r = n result bit for bit, and
    the oracle's."""
    dev = _dev()
    n, w, g = 300, 16, 2
    q, k, v = synth.qkv(1, 2, n, 128, dtype, seed=96, device=dev)
    outs = []
    for r in (n, 2 ** 20, 2 ** 30):
        if kind == "dilated":
            outs.append(swa.dilated_prefill(q, k, v, w=w, r=r, return_lse=True))
        else:
            outs.append(swa.landmark_prefill(q, k, v, w=w, g=g, r=r, sink_bias=1.0, return_lse=True))
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    gg, beta = (0, 0.0) if kind == "dilated" else (g, 1.0)
    _check(q, k, v, outs[-1][0], outs[-1][1], kind, w, gg, 2 ** 30, beta)
