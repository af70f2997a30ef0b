"""Chunked prefill against the rolling cache, and the LSE merge, on the HIP
path (through the C ABI) against the fp64 oracle.

The chunk's rows must equal rows p0 .. p0+T-1 of the oracle's prefill over
the whole logical sequence ("Sliding Window and Sparse Attention, from
Longformer to CSA2", s2; "Local and Sparse Attention: Reading Fewer Token
Positions", Figure 4 and its multi-token buffers).  The cache is filled by
kv_append from NaN-poisoned memory, so a read of any row the cache does not
hold shows up as NaN, masked or not (0 x NaN is NaN in the value product).
Tolerances: fp32 1e-4, bf16 2e-2 max-abs (outputs and LSE).
"""
import math

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


def _problem(p0s, T, H, Hkv, d, w, g, dtype, seed):
    """Logical K/V sequences (CPU), the chunk's q, and NaN-poisoned caches
    filled by kv_append with positions 0 .. p0-1 of each batch entry."""
    dev = _dev()
    B = len(p0s)
    n_tot = max(p0s) + T
    kseq = synth.normal((B, Hkv, n_tot, d), seed=seed, dtype=dtype)
    vseq = synth.normal((B, Hkv, n_tot, d), seed=seed + 1, dtype=dtype)
    q = synth.normal((B, H, T, d), seed=seed + 2, dtype=dtype)
    kc = torch.full((B, Hkv, g + w, d), float("nan"), dtype=dtype, device=dev)
    vc = torch.full_like(kc, float("nan"))
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    for b, p0 in enumerate(p0s):
        if p0 > 0:
            swa.kv_append(kc[b:b + 1], vc[b:b + 1], kseq[b:b + 1, :, :p0].contiguous().to(dev),
                          vseq[b:b + 1, :, :p0].contiguous().to(dev), zero, w=w, g=g)
    kn = torch.stack([kseq[b, :, p0:p0 + T] for b, p0 in enumerate(p0s)]).contiguous()
    vn = torch.stack([vseq[b, :, p0:p0 + T] for b, p0 in enumerate(p0s)]).contiguous()
    pos = torch.tensor(p0s, dtype=torch.int64, device=dev)
    return q, kseq, vseq, kn, vn, kc, vc, pos


def _oracle_rows(orc, q, kseq, vseq, p0s, T, w, g, beta):
    """Rows p0 .. p0+T-1 of the oracle's prefill over each logical sequence."""
    out_o, out_l = [], []
    H, d = q.shape[1], q.shape[3]
    for b, p0 in enumerate(p0s):
        qf = torch.zeros(H, p0 + T, d, dtype=torch.float64)
        qf[:, p0:] = q[b].double()
        ro, rl = orc.prefill(qf, kseq[b, :, :p0 + T], vseq[b, :, :p0 + T], w=w, g=g, beta=beta,
                             rows=np.arange(p0, p0 + T))
        out_o.append(ro)
        out_l.append(rl)
    return np.stack(out_o), np.stack(out_l)


CASES = [
    # (w, g, beta, T, p0s): first chunk, p0 below g, inside the first window,
    # the ring's wrap inside a key tile, long histories, T below one tile
    (64, 4, 0.5, 100, [0, 1, 3, 37, 64, 130, 1000]),
    (100, 0, 0.0, 257, [0, 50, 99, 100, 371]),
    (8, 2, -1.0, 33, [0, 5, 9, 200]),
    (300, 4, 2.0, 64, [10, 299, 300, 301, 1234]),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w,g,beta,T,p0s", CASES)
def test_chunk_vs_oracle(orc, dtype, d, w, g, beta, T, p0s):
    dev = _dev()
    H = Hkv = 2
    q, kseq, vseq, kn, vn, kc, vc, pos = _problem(p0s, T, H, Hkv, d, w, g, dtype, seed=71)
    o, lse = swa.chunk_prefill(q.to(dev), kn.to(dev), vn.to(dev), kc, vc, pos, w=w, g=g, sink_bias=beta,
                               return_lse=True)
    torch.cuda.synchronize()
    ro, rl = _oracle_rows(orc, q, kseq, vseq, p0s, T, w, g, beta)
    go = o.float().cpu().numpy()
    gate(go, ro, dtype, f"chunk w={w} g={g} T={T} d={d}")
    gate(lse.cpu().numpy(), rl, dtype, "chunk lse")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_gqa_vs_oracle(orc, dtype):
    dev = _dev()
    H, Hkv, d, w, g, T, p0s = 8, 2, 128, 96, 4, 150, [0, 70, 500]
    q, kseq, vseq, kn, vn, kc, vc, pos = _problem(p0s, T, H, Hkv, d, w, g, dtype, seed=72)
    o = swa.chunk_prefill(q.to(dev), kn.to(dev), vn.to(dev), kc, vc, pos, w=w, g=g, sink_bias=1.0)
    torch.cuda.synchronize()
    ro, _ = _oracle_rows(orc, q, kseq, vseq, p0s, T, w, g, 1.0)
    gate(o.float().cpu().numpy(), ro, dtype, "chunk gqa")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_random_shapes(orc, dtype):
    """Seeded random chunks: windows narrower and wider than a key tile and
    than the chunk, sink counts below, at and above a tile, chunk lengths
    from one row to several blocks, positions before, at and past the first
    ring wrap, grouped heads and both head sizes; every row of each chunk
    against the oracle."""
    dev = _dev()
    rng = np.random.default_rng(2024)
    for case in range(6):
        w = int(rng.integers(1, 300))
        g = int(rng.choice([0, 1, 4, 64, 70]))
        T = int(rng.integers(1, 300))
        p0s = sorted(int(x) for x in rng.integers(0, 3 * w + 200, size=2))
        d = int(rng.choice([64, 128]))
        H, Hkv = [(2, 2), (4, 2), (3, 1)][case % 3]
        beta = float(rng.uniform(-2.0, 4.0))
        print(f"case {case}: w={w} g={g} T={T} p0s={p0s} d={d} H={H}/{Hkv} {dtype}", flush=True)
        q, kseq, vseq, kn, vn, kc, vc, pos = _problem(p0s, T, H, Hkv, d, w, g, dtype, seed=300 + 7 * case)
        o, lse = swa.chunk_prefill(q.to(dev), kn.to(dev), vn.to(dev), kc, vc, pos, w=w, g=g, sink_bias=beta,
                                   return_lse=True)
        torch.cuda.synchronize()
        ro, rl = _oracle_rows(orc, q, kseq, vseq, p0s, T, w, g, beta)
        gate(o.float().cpu().numpy(), ro, dtype, f"chunk case {case}")
        gate(lse.cpu().numpy(), rl, dtype, f"chunk case {case} lse")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_partials_merge_to_full(orc, dtype):
    """Cache-only and chunk-only partials merged by swa_lse_merge equal the
    full chunk result and the oracle; a row with no cache key has o = 0 and
    lse = -inf in the cache partial."""
    dev = _dev()
    w, g, beta, T, p0s = 64, 4, 1.5, 200, [0, 3, 40, 130, 700]
    q, kseq, vseq, kn, vn, kc, vc, pos = _problem(p0s, T, 2, 2, 128, w, g, dtype, seed=73)
    args = (q.to(dev), kn.to(dev), vn.to(dev), kc, vc, pos)
    oc, lc = swa.chunk_prefill(*args, w=w, g=g, sink_bias=beta, keys="cache", return_lse=True)
    on, ln = swa.chunk_prefill(*args, w=w, g=g, sink_bias=beta, keys="chunk", return_lse=True)
    om, lm = swa.lse_merge(oc, lc, on, ln)
    torch.cuda.synchronize()
    ro, rl = _oracle_rows(orc, q, kseq, vseq, p0s, T, w, g, beta)
    gate(om.float().cpu().numpy(), ro, dtype, "chunk partials merged")
    gate(lm.cpu().numpy(), rl, dtype, "chunk partials merged lse")
    # rows whose window lies inside the chunk and whose sinks are too (or g = 0 reached): no cache key
    lc_h, oc_h = lc.cpu().numpy(), oc.float().cpu().numpy()
    for b, p0 in enumerate(p0s):
        for i in range(T):
            P = p0 + i
            has_cache = p0 > 0 and (P - w + 1 <= p0 - 1 or min(g, p0) > 0)
            if not has_cache:
                assert np.all(np.isneginf(lc_h[b, :, i])) and np.all(oc_h[b, :, i] == 0)
            else:
                assert np.all(np.isfinite(lc_h[b, :, i]))


def test_lse_merge_vs_oracle(orc):
    dev = _dev()
    rng = np.random.default_rng(74)
    rows, d = 1000, 128
    oa, ob = rng.standard_normal((rows, d)), rng.standard_normal((rows, d))
    la, lb = rng.standard_normal(rows) * 4, rng.standard_normal(rows) * 4
    la[::7] = -np.inf
    lb[::11] = -np.inf
    ro, rl = oracle.lse_merge(oa, la, ob, lb)
    for dtype, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2)):
        ta, tb = torch.tensor(oa).to(dtype).to(dev), torch.tensor(ob).to(dtype).to(dev)
        o, lse = swa.lse_merge(ta, torch.tensor(la, dtype=torch.float32, device=dev), tb,
                               torch.tensor(lb, dtype=torch.float32, device=dev))
        torch.cuda.synchronize()
        # the oracle merges the same (rounded) inputs
        ro2, _ = oracle.lse_merge(ta.double().cpu().numpy(), la, tb.double().cpu().numpy(), lb)
        assert float(np.max(np.abs(o.double().cpu().numpy() - ro2))) <= tol
        gl = lse.cpu().numpy()
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(gl), fin)
        assert float(np.max(np.abs(gl[fin] - rl[fin]))) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunks_reproduce_prefill(orc, dtype):
    """A sequence processed as chunks (chunk prefill, then append) equals the
    one-shot prefill (GPU) and the oracle."""
    dev = _dev()
    B, H, n, d, w, g, beta = 1, 2, 1000, 128, 256, 4, 1.0
    q, k, v = synth.qkv(B, H, n, d, dtype, seed=75, device=dev)
    full = swa.prefill(q, k, v, w=w, g=g, sink_bias=beta)
    kc = torch.full((B, H, g + w, d), float("nan"), dtype=dtype, device=dev)
    vc = torch.full_like(kc, float("nan"))
    outs, p0 = [], 0
    for T in (300, 1, 299, 400):
        pos = torch.full((B,), p0, dtype=torch.int64, device=dev)
        sl = slice(p0, p0 + T)
        outs.append(swa.chunk_prefill(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(),
                                      kc, vc, pos, w=w, g=g, sink_bias=beta))
        swa.kv_append(kc, vc, k[:, :, sl].contiguous(), v[:, :, sl].contiguous(), pos, w=w, g=g)
        p0 += T
    chunked = torch.cat(outs, dim=2)
    torch.cuda.synchronize()
    assert torch.isfinite(chunked.float()).all()
    assert float((chunked.float() - full.float()).abs().max()) <= _tol(dtype)
    ro, _ = orc.prefill(q[0].cpu(), k[0].cpu(), v[0].cpu(), w=w, g=g, beta=beta)
    assert float(np.max(np.abs(chunked[0].float().cpu().numpy() - ro))) <= _tol(dtype)


def test_chunk_negative_position_gives_nan():
    dev = _dev()
    B, H, T, d, w, g = 2, 2, 40, 128, 16, 4
    q = synth.normal((B, H, T, d), seed=1, dtype=torch.bfloat16, device=dev)
    kn = synth.normal((B, H, T, d), seed=2, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(B, H, g + w, d, dtype=torch.bfloat16, device=dev)
    pos = torch.tensor([-3, 0], dtype=torch.int64, device=dev)
    o = swa.chunk_prefill(q, kn, kn, kc, kc, pos, w=w, g=g)
    torch.cuda.synchronize()
    assert torch.isnan(o[0].float()).all() and torch.isfinite(o[1].float()).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_far_positions_match_near_ones(dtype):
    """A chunk at position p0 and at p0 + k w (k w a multiple of the 64-key
    tile, p0 past w + g) reads the same ring rows and sink rows through the
    same tiles, so the outputs agree bit for bit; p0 + k w is put at the
    last accepted position (pos + t = INT_MAX - 1024), where every position
    sum of the tile arithmetic must still be an int.  One past it gives NaN
    rows."""
    dev = _dev()
    B, H, T, d, w, g, beta = 1, 2, 100, 128, 128, 4, 1.5
    q = synth.normal((B, H, T, d), seed=11, dtype=dtype, device=dev)
    kn = synth.normal((B, H, T, d), seed=12, dtype=dtype, device=dev)
    vn = synth.normal((B, H, T, d), seed=13, dtype=dtype, device=dev)
    kc = synth.normal((B, H, g + w, d), seed=14, dtype=dtype, device=dev)
    vc = synth.normal((B, H, g + w, d), seed=15, dtype=dtype, device=dev)
    last = 2 ** 31 - 1 - 1024 - T             # the largest accepted p0
    far = last - (last - 1000) % w             # far = near (mod w), near = 1000 + ...
    near = far % w + 4 * w                     # past w + g, same residue mod w (w is a multiple of 64)
    assert (far - near) % w == 0 and (far - near) % 64 == 0 and far <= last and near > w + g
    print(f"chunk at {near} and at {far} (last accepted {last})", flush=True)
    outs = []
    for p0 in (near, far):
        pos = torch.tensor([p0], dtype=torch.int64, device=dev)
        outs.append(swa.chunk_prefill(q, kn, vn, kc, vc, pos, w=w, g=g, sink_bias=beta, return_lse=True))
    pos = torch.tensor([last + 1], dtype=torch.int64, device=dev)
    over = swa.chunk_prefill(q, kn, vn, kc, vc, pos, w=w, g=g, sink_bias=beta)
    torch.cuda.synchronize()
    (o_near, l_near), (o_far, l_far) = outs
    assert torch.isfinite(o_near.float()).all()
    assert torch.equal(o_near, o_far) and torch.equal(l_near, l_far)
    assert torch.isnan(over.float()).all()


def test_chunk_full_size_sampled(orc):
    """Mistral-shaped chunk: 32 query heads over 8 key/value heads, d=128,
    w=4096, g=4, a 4096-token chunk at position 16384 against a full ring of
    random rows; 48 sampled (head, row) pairs against the oracle, given the
    rows the cache model says hold each attended position."""
    dev = _dev()
    B, H, Hkv, T, d, w, g, p0 = 1, 32, 8, 4096, 128, 4096, 4, 16384
    q, kn, vn = synth.qkv(B, H, T, d, torch.bfloat16, seed=76, device=dev, kv_heads=Hkv)
    kc = synth.normal((B, Hkv, g + w, d), seed=77, dtype=torch.bfloat16, device=dev)
    vc = synth.normal((B, Hkv, g + w, d), seed=78, dtype=torch.bfloat16, device=dev)
    pos = torch.tensor([p0], dtype=torch.int64, device=dev)
    o, lse = swa.chunk_prefill(q, kn, vn, kc, vc, pos, w=w, g=g, return_lse=True)
    torch.cuda.synchronize()
    cpos, crow = cache_model.logical_rows(p0 - 1, w, g)
    row_of = dict(zip(cpos.tolist(), crow.tolist()))
    rng = np.random.default_rng(76)
    samples = sorted({(int(h), int(i)) for h, i in zip(rng.integers(0, H, 48), rng.integers(0, T, 48))})
    nk = g + w
    qs, ps, kps, ks, vs = [], [], [], [], []
    kc_h, vc_h, kn_h, vn_h = (t[0].double().cpu() for t in (kc, vc, kn, vn))
    for h, i in samples:
        j = oracle.kv_head_of(h, H, Hkv)
        P = p0 + i
        att = list(range(max(0, P - w + 1), P + 1)) + [s for s in range(min(g, P + 1)) if s < P - w + 1]
        kk = torch.zeros(nk, d, dtype=torch.float64)
        vv = torch.zeros(nk, d, dtype=torch.float64)
        kp = np.full(nk, -1, dtype=np.int64)
        for r, s in enumerate(att):
            kp[r] = s
            if s >= p0:
                kk[r], vv[r] = kn_h[j, s - p0], vn_h[j, s - p0]
            else:
                kk[r], vv[r] = kc_h[j, row_of[s]], vc_h[j, row_of[s]]
        qs.append(q[0, h, i].double().cpu()); ps.append(P); kps.append(kp); ks.append(kk); vs.append(vv)
    ro, rl = orc.decode(torch.stack(qs), ps, np.stack(kps), torch.stack(ks), torch.stack(vs), w=w, g=g)
    go = torch.stack([o[0, h, i] for h, i in samples]).float().cpu().numpy()
    gl = torch.stack([lse[0, h, i] for h, i in samples]).cpu().numpy()
    gate(go, ro, torch.bfloat16, f"chunk full size, {len(samples)} sampled rows")
    gate(gl, rl, torch.bfloat16, "chunk full size lse")
