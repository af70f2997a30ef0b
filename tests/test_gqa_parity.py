"""Grouped-query attention on the HIP path (through the C ABI) against the oracle.

Query head h of H reads key/value head h // (H / Hkv) (consecutive groups;
"Sliding Window and Sparse Attention, from Longformer to CSA2", s10 glossary,
GQA).  Same tolerances as the multi-head tests: fp32 1e-4, bf16 2e-2 max-abs.
Prefill is also held bit-exact to the multi-head call on key/value heads
copied out per query head (the kernel reads the same rows either way); decode
covers one, two, four and eight query heads per workgroup, group sizes that
are not powers of two, and the split-and-merge path.
"""
import numpy as np
import pytest
import torch

import block_sparse_causal_band_amd as swa
import oracle
from block_sparse_causal_band_amd import synth
from oracle import cache_model
from tests.parity import gate

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda")


def _tol(dtype):
    return BF16_TOL if dtype == torch.bfloat16 else F32_TOL


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(8, 2), (8, 1), (6, 3), (4, 4)])
def test_prefill_gqa_vs_oracle(orc, dtype, d, H, Hkv):
    """n = 300 spans several query and key tiles and ends in a ragged one."""
    dev = _dev()
    B, n, w, g, beta = 2, 300, 70, 4, 1.0
    q, k, v = synth.qkv(B, H, n, d, dtype, seed=61, kv_heads=Hkv)
    o, lse = swa.prefill(q.to(dev), k.to(dev), v.to(dev), w=w, g=g, sink_bias=beta, return_lse=True)
    torch.cuda.synchronize()
    for b in range(B):
        ro, rl = orc.prefill(q[b], k[b], v[b], w=w, g=g, beta=beta)
        go = o[b].float().cpu().numpy()
        gate(go, ro, dtype, f"gqa prefill b={b} H={H} Hkv={Hkv} d={d}")
        gate(lse[b].cpu().numpy(), rl, dtype, "gqa prefill lse")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("H,Hkv", [(32, 8), (16, 1)])
def test_prefill_gqa_equals_expanded_heads(dtype, H, Hkv):
    dev = _dev()
    B, n, d, w, g = 1, 1000, 128, 256, 4
    q, k, v = synth.qkv(B, H, n, d, dtype, seed=62, device=dev, kv_heads=Hkv)
    idx = torch.tensor([oracle.kv_head_of(h, H, Hkv) for h in range(H)], device=dev)
    ke, ve = k.index_select(1, idx).contiguous(), v.index_select(1, idx).contiguous()
    a, la = swa.prefill(q, k, v, w=w, g=g, sink_bias=0.5, return_lse=True)
    b, lb = swa.prefill(q, ke, ve, w=w, g=g, sink_bias=0.5, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)



def test_prefill_gqa_full_size_sampled(orc):
    """The grouped-query prefill workload at full size (batch 1, 32 query
    heads over 8 key/value heads, n=16384, d=128, w=4096, bf16), as timed:
    sampled rows (the band edges, the tail and 40 random rows) of query heads
    at the start, middle and end of groups, each against the oracle over its
    own key/value head."""
    dev = _dev()
    B, H, Hkv, n, d, w, g = 1, 32, 8, 16384, 128, 4096, 0
    q, k, v = synth.qkv(B, H, n, d, torch.bfloat16, seed=9, device=dev, kv_heads=Hkv)
    o, lse = swa.prefill(q, k, v, w=w, g=g, sink_bias=0.0, return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    fixed = [0, 1, 63, 64, 127, 128, w - 1, w, w + 127, n - 129, n - 128, n - 1]
    rows = sorted(set(fixed + rng.choice(n, size=40, replace=False).tolist()))
    for h in (0, 3, 13, 31):
        j = oracle.kv_head_of(h, H, Hkv)
        ro, rl = orc.prefill(q[0, h].cpu(), k[0, j].cpu(), v[0, j].cpu(), w=w, g=g, beta=0.0, rows=rows)
        gate(o[0, h].float().cpu().numpy()[rows], ro, q.dtype, f"gqa prefill full size, head {h} (kv {j})")
        gate(lse[0, h].cpu().numpy()[rows], rl, q.dtype, f"gqa prefill lse, head {h}")


def _decode_gqa_vs_oracle(orc, q, kc, vc, pos, w, g, beta, units=None):
    B, H, d = q.shape
    Hkv = kc.shape[1]
    o, lse = swa.decode(q, kc, vc, pos, w=w, g=g, sink_bias=beta, return_lse=True)
    torch.cuda.synchronize()
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]
    pos_h = pos.cpu().tolist()
    nk = g + w
    qs, ps, kps, ks, vs = [], [], [], [], []
    for b, h in units:
        p = pos_h[b]
        j = oracle.kv_head_of(h, H, Hkv)
        positions, rows = cache_model.logical_rows(p, w, g)
        kp = np.full(nk, -1, dtype=np.int64)
        kp[:len(positions)] = positions
        rows_t = torch.as_tensor(rows, device=kc.device)
        kk = torch.zeros(nk, d, dtype=torch.float64)
        vv = torch.zeros(nk, d, dtype=torch.float64)
        kk[:len(rows)] = kc[b, j].index_select(0, rows_t).double().cpu()
        vv[:len(rows)] = vc[b, j].index_select(0, rows_t).double().cpu()
        qs.append(q[b, h].double().cpu()); ps.append(p); kps.append(kp); ks.append(kk); vs.append(vv)
    ro, rl = orc.decode(torch.stack(qs), ps, np.stack(kps), torch.stack(ks), torch.stack(vs), w=w, g=g, beta=beta)
    go = torch.stack([o[b, h] for b, h in units]).float().cpu().numpy()
    gl = torch.stack([lse[b, h] for b, h in units]).cpu().numpy()
    err, _ = gate(go, ro, q.dtype, f"gqa decode H={H} Hkv={Hkv} w={w} g={g}")
    gate(gl, rl, q.dtype, "gqa decode lse")
    return err


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(8, 8), (8, 4), (8, 2), (8, 1), (12, 4), (32, 2)])
def test_decode_gqa_vs_oracle(orc, dtype, d, H, Hkv):
    """Group sizes 1, 2, 4, 8, 3 and 16 (two workgroups of eight heads per
    key/value head); positions before, at and past the ring's wrap."""
    dev = _dev()
    w, g = 100, 4
    positions = [0, 3, 50, 99, 100, 104, 517]
    B = len(positions)
    q, kc, vc, _ = synth.decode_problem(B, H, d, g + w, 0, 0, dtype, seed=63, device=dev, kv_heads=Hkv)
    pos = torch.tensor(positions, dtype=torch.int64, device=dev)
    _decode_gqa_vs_oracle(orc, q, kc, vc, pos, w, g, 0.5)


@pytest.mark.parametrize("B,H,Hkv", [(1, 8, 1), (2, 32, 8), (3, 64, 8), (64, 32, 8)])
def test_decode_gqa_split_and_unsplit(orc, B, H, Hkv):
    """Few workgroups split the cache and merge by LSE; many do not."""
    dev = _dev()
    w, g, d = 4096, 4, 128
    q, kc, vc, pos = synth.decode_problem(B, H, d, g + w, w, 40000, torch.bfloat16, seed=64, device=dev,
                                          kv_heads=Hkv)
    rng = np.random.default_rng(64)
    units = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, B, 48), rng.integers(0, H, 48))})
    _decode_gqa_vs_oracle(orc, q, kc, vc, pos, w, g, 0.0, units=units)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_random_shapes(orc, dtype):
    """Seeded random decode problems: ring sizes, sink counts, head groupings
    (one to eight query heads per key/value head), head sizes and positions
    before, at and far past the ring's wrap."""
    dev = _dev()
    rng = np.random.default_rng(78)
    for case in range(8):
        w = int(rng.integers(1, 300))
        g = int(rng.integers(0, 20))
        d = int(rng.choice([64, 128]))
        H, Hkv = [(1, 1), (4, 4), (8, 2), (8, 1), (6, 3), (16, 2), (2, 1), (5, 5)][case]
        B = int(rng.integers(1, 5))
        q, kc, vc, _ = synth.decode_problem(B, H, d, g + w, 0, 0, dtype, seed=200 + case, device=dev, kv_heads=Hkv)
        positions = [int(x) for x in rng.integers(0, 4 * w + g + 2, B)]
        pos = torch.tensor(positions, dtype=torch.int64, device=dev)
        _decode_gqa_vs_oracle(orc, q, kc, vc, pos, w, g, float(rng.uniform(-1.0, 3.0)))


def test_decode_gqa_through_appended_cache(orc):
    """kv_append writes Hkv heads; decode of H query heads reads them."""
    dev = _dev()
    B, H, Hkv, d, w, g, n = 2, 8, 2, 128, 64, 4, 150
    kseq = synth.normal((B, Hkv, n, d), seed=65, dtype=torch.bfloat16, device=dev)
    vseq = synth.normal((B, Hkv, n, d), seed=66, dtype=torch.bfloat16, device=dev)
    q = synth.normal((B, H, d), seed=67, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(B, Hkv, g + w, d, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    swa.kv_append(kc, vc, kseq, vseq, torch.zeros(B, dtype=torch.int64, device=dev), w=w, g=g)
    pos = torch.full((B,), n - 1, dtype=torch.int64, device=dev)
    o = swa.decode(q, kc, vc, pos, w=w, g=g, sink_bias=2.0).float().cpu().numpy()
    for b in range(B):
        qseq = torch.zeros(H, n, d, dtype=torch.float64)
        qseq[:, n - 1] = q[b].double().cpu()
        ro, _ = orc.prefill(qseq, kseq[b].cpu(), vseq[b].cpu(), w=w, g=g, beta=2.0, rows=[n - 1])
        assert float(np.max(np.abs(o[b] - ro[:, 0]))) <= BF16_TOL


def test_gqa_rejects_bad_kv_heads():
    dev = _dev()
    q = torch.zeros(1, 6, 64, 64, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(Exception):
        swa.prefill(q, k, k, w=8, g=0)


def test_decode_gqa_negative_position_and_determinism():
    """The matrix-core decode: a negative position gives NaN rows, other rows
    stay finite, and two launches agree bit for bit."""
    dev = _dev()
    q, kc, vc, _ = synth.decode_problem(2, 8, 128, 520, 0, 0, torch.bfloat16, seed=68, device=dev, kv_heads=2)
    pos = torch.tensor([-1, 700], dtype=torch.int64, device=dev)
    a = swa.decode(q, kc, vc, pos, w=516, g=4)
    b = swa.decode(q, kc, vc, pos, w=516, g=4)
    torch.cuda.synchronize()
    assert torch.isnan(a[0].float()).all() and torch.isfinite(a[1].float()).all()
    assert torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_gqa_ignores_unwritten_rows(orc, dtype):
    """NaN in never-written ring slots and sink rows does not reach grouped
    decode outputs at early positions."""
    dev = _dev()
    w, g, d, H, Hkv = 64, 4, 128, 8, 2
    positions = [0, 1, 5, 30, 62]
    B, n = len(positions), max(positions) + 1
    kseq = synth.normal((B, Hkv, n, d), seed=69, dtype=dtype, device="cpu")
    vseq = synth.normal((B, Hkv, n, d), seed=70, dtype=dtype, device="cpu")
    q = synth.normal((B, H, d), seed=71, dtype=dtype, device="cpu").to(dev)
    kc = torch.full((B, Hkv, g + w, d), float("nan"), dtype=dtype, device=dev)
    vc = torch.full_like(kc, float("nan"))
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    for b, p in enumerate(positions):
        swa.kv_append(kc[b:b + 1], vc[b:b + 1], kseq[b:b + 1, :, :p + 1].contiguous().to(dev),
                      vseq[b:b + 1, :, :p + 1].contiguous().to(dev), zero, w=w, g=g)
    pos = torch.tensor(positions, dtype=torch.int64, device=dev)
    _decode_gqa_vs_oracle(orc, q, kc, vc, pos, w, g, 0.0)
