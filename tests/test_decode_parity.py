"""HIP kv_append and decode kernels (through the C ABI) against the oracle.

kv_append must equal the token-by-token cache model bit for bit.  decode is
compared with the oracle's decode over the logical sequence (fp32 1e-4,
bf16 2e-2 max-abs); the oracle never reads the cache layout itself.
"""
import numpy as np
import pytest
import torch

import block_sparse_causal_band_amd as swa
from block_sparse_causal_band_amd import synth
from oracle import cache_model
from tests.parity import gate

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w,g,T,starts", [
    (8, 0, 1, [0, 5, 17]), (8, 4, 3, [0, 2, 40]), (8, 4, 13, [0, 1, 9]), (5, 3, 30, [0, 2, 7]),
    (64, 4, 64, [0, 64, 1000]), (16, 0, 40, [3, 0, 100]),
])
def test_kv_append_bit_exact(dtype, d, w, g, T, starts):
    dev = _dev()
    B, H = len(starts), 2
    kc0 = synth.normal((B, H, g + w, d), seed=1, dtype=dtype)
    vc0 = synth.normal((B, H, g + w, d), seed=2, dtype=dtype)
    kn = synth.normal((B, H, T, d), seed=3, dtype=dtype)
    vn = synth.normal((B, H, T, d), seed=4, dtype=dtype)
    pos = torch.tensor(starts, dtype=torch.int64)
    ref_k, ref_v = kc0.clone(), vc0.clone()
    cache_model.append(ref_k, ref_v, kn, vn, pos.tolist(), w, g)
    gk, gv = kc0.to(dev), vc0.to(dev)
    swa.kv_append(gk, gv, kn.to(dev), vn.to(dev), pos.to(dev), w=w, g=g)
    torch.cuda.synchronize()
    assert torch.equal(gk.cpu(), ref_k) and torch.equal(gv.cpu(), ref_v)


@pytest.mark.parametrize("fp8", [False, True])
def test_kv_append_positions_near_int64_max(fp8):
    """The last accepted start (pos + t_new = INT64_MAX) writes the ring rows
    the cache model gives for those positions; one further (the last token
    would wrap past INT64_MAX) leaves the entry untouched, as a negative
    position does."""
    dev = _dev()
    B, H, T, d, w, g = 3, 2, 5, 128, 16, 4
    top = 2 ** 63 - 1
    starts = [top - T, top - T + 1, 7]
    kc0 = synth.normal((B, H, g + w, d), seed=21, dtype=torch.bfloat16)
    vc0 = synth.normal((B, H, g + w, d), seed=22, dtype=torch.bfloat16)
    kn = synth.normal((B, H, T, d), seed=23, dtype=torch.bfloat16)
    vn = synth.normal((B, H, T, d), seed=24, dtype=torch.bfloat16)
    pos = torch.tensor(starts, dtype=torch.int64)
    print(f"kv_append{'_fp8' if fp8 else ''} starts {starts}", flush=True)
    if fp8:
        scale = torch.full((B, H), 0.05, dtype=torch.float32)
        codes_k = torch.zeros(B, H, g + w, d, dtype=torch.uint8, device=dev)
        codes_v = torch.zeros_like(codes_k)
        swa.kv_append_fp8(codes_k, codes_v, kn.to(dev), vn.to(dev), pos.to(dev), scale.to(dev), scale.to(dev), w=w, g=g)
        torch.cuda.synchronize()
        written = (codes_k.cpu() != 0).flatten(2).any(-1)  # [B, H]: rows written per entry
        assert written[0].all() and not written[1].any() and written[2].all()
        return
    expect_k, expect_v = kc0.clone(), vc0.clone()  # entry 1 stays as it was
    for b in (0, 2):
        rk, rv = kc0[b:b + 1].clone(), vc0[b:b + 1].clone()
        cache_model.append(rk, rv, kn[b:b + 1], vn[b:b + 1], [starts[b]], w, g)
        expect_k[b], expect_v[b] = rk[0], rv[0]
    gk, gv = kc0.to(dev), vc0.to(dev)
    swa.kv_append(gk, gv, kn.to(dev), vn.to(dev), pos.to(dev), w=w, g=g)
    torch.cuda.synchronize()
    assert torch.equal(gk.cpu(), expect_k) and torch.equal(gv.cpu(), expect_v)


def _decode_vs_oracle(orc, q, kc, vc, pos, w, g, beta, units=None, tol=None):
    """GPU decode vs the oracle; the oracle receives logical rows (position,
    k, v) that the cache model says the cache supplies for each query."""
    B, H, d = q.shape
    o, lse = swa.decode(q, kc, vc, pos, w=w, g=g, sink_bias=beta, return_lse=True)
    torch.cuda.synchronize()
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]
    if tol is None:
        tol = BF16_TOL if q.dtype == torch.bfloat16 else F32_TOL
    pos_h = pos.cpu().tolist()
    qs, ps, kps, ks, vs = [], [], [], [], []
    nk = g + w
    for b, h in units:
        p = pos_h[b]
        positions, rows = cache_model.logical_rows(p, w, g)
        kp = np.full(nk, -1, dtype=np.int64)
        kp[:len(positions)] = positions
        rows_t = torch.as_tensor(rows, device=kc.device)
        kk = torch.zeros(nk, d, dtype=torch.float64)
        vv = torch.zeros(nk, d, dtype=torch.float64)
        kk[:len(rows)] = kc[b, h].index_select(0, rows_t).double().cpu()
        vv[:len(rows)] = vc[b, h].index_select(0, rows_t).double().cpu()
        qs.append(q[b, h].double().cpu()); ps.append(p); kps.append(kp); ks.append(kk); vs.append(vv)
    ro, rl = orc.decode(torch.stack(qs), ps, np.stack(kps), torch.stack(ks), torch.stack(vs),
                        w=w, g=g, beta=beta)
    go = torch.stack([o[b, h] for b, h in units]).float().cpu().numpy()
    gl = torch.stack([lse[b, h] for b, h in units]).cpu().numpy()
    err, _ = gate(go, ro, q.dtype, f"decode {tuple(q.shape)} w={w} g={g}", tol=tol)
    gate(gl, rl, q.dtype, "decode lse", tol=(1e-4 if q.dtype == torch.float32 else 2e-2))
    return err


EDGE_POS = lambda w, g: sorted({0, 1, 2, 3, g, w - 2, w - 1, w, w + 1, w + 2, w + g - 1, w + g, 3 * w + 7})


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w,g,beta", [(16, 0, 0.0), (16, 4, 0.0), (100, 4, 4.0), (7, 9, -1.0), (1, 2, 1.0)])
def test_decode_through_appended_cache(orc, dtype, d, w, g, beta):
    """Fill the cache by kv_append with positions 0..p of a logical sequence,
    then decode at p: every edge position of the ring and the sinks."""
    dev = _dev()
    positions = [p for p in EDGE_POS(w, g) if p >= 0]
    B, H = len(positions), 3
    n = max(positions) + 1
    kseq = synth.normal((B, H, n, d), seed=31, dtype=dtype, device="cpu")
    vseq = synth.normal((B, H, n, d), seed=32, dtype=dtype, device="cpu")
    q = synth.normal((B, H, d), seed=33, dtype=dtype, device="cpu").to(dev)
    kc = torch.zeros(B, H, g + w, d, dtype=dtype, device=dev)
    vc = torch.zeros_like(kc)
    # append each batch entry's prefix 0..p in one multi-token call
    for b, p in enumerate(positions):
        one = torch.zeros(1, dtype=torch.int64, device=dev)
        swa.kv_append(kc[b:b + 1], vc[b:b + 1], kseq[b:b + 1, :, :p + 1].contiguous().to(dev),
                      vseq[b:b + 1, :, :p + 1].contiguous().to(dev), one, w=w, g=g)
    pos = torch.tensor(positions, dtype=torch.int64, device=dev)
    _decode_vs_oracle(orc, q, kc, vc, pos, w, g, beta)
    # and equals row p of the oracle's prefill over the logical sequence
    o_gpu = swa.decode(q, kc, vc, pos, w=w, g=g, sink_bias=beta).float().cpu().numpy()
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    for b, p in enumerate(positions):
        qseq = torch.zeros(H, p + 1, d, dtype=torch.float64)
        qseq[:, p] = q[b].double().cpu()
        ro, _ = orc.prefill(qseq, kseq[b, :, :p + 1], vseq[b, :, :p + 1], w=w, g=g, beta=beta, rows=[p])
        assert float(np.max(np.abs(o_gpu[b] - ro[:, 0]))) <= tol


@pytest.mark.parametrize("B,H", [(1, 1), (2, 3), (8, 128)])
def test_decode_split_and_unsplit(orc, B, H):
    """Few (batch, head) pairs split the cache over workgroups and merge by
    LSE; many pairs do not.  Both paths against the oracle."""
    dev = _dev()
    w, g, d = 700, 4, 128
    q, kc, vc, pos = synth.decode_problem(B, H, d, g + w, w, 5 * w, torch.bfloat16, seed=41, device=dev)
    units = [(b, h) for b in range(B) for h in range(H)][:64]
    _decode_vs_oracle(orc, q, kc, vc, pos, w, g, 0.5, units=units)


def test_decode_negative_position_gives_nan():
    dev = _dev()
    q, kc, vc, _ = synth.decode_problem(2, 2, 128, 20, 16, 16, torch.bfloat16, seed=1, device=dev)
    pos = torch.tensor([-1, 30], dtype=torch.int64, device=dev)
    o = swa.decode(q, kc, vc, pos, w=16, g=4)
    torch.cuda.synchronize()
    assert torch.isnan(o[0].float()).all() and torch.isfinite(o[1].float()).all()


def test_decode_equals_prefill_row():
    """Decode at p over a cache filled by kv_append equals prefill row p (GPU vs GPU)."""
    dev = _dev()
    B, H, n, d, w, g = 1, 4, 1500, 128, 512, 4
    q, k, v = synth.qkv(B, H, n, d, torch.bfloat16, seed=51, device=dev)
    o_pre = swa.prefill(q, k, v, w=w, g=g, sink_bias=4.0)
    kc = torch.zeros(B, H, g + w, d, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    zero = torch.zeros(B, dtype=torch.int64, device=dev)
    swa.kv_append(kc, vc, k, v, zero, w=w, g=g)
    pos = torch.full((B,), n - 1, dtype=torch.int64, device=dev)
    o_dec = swa.decode(q[:, :, n - 1].contiguous(), kc, vc, pos, w=w, g=g, sink_bias=4.0)
    torch.cuda.synchronize()
    assert float((o_dec.float() - o_pre[:, :, n - 1].float()).abs().max()) <= BF16_TOL


def test_decode_full_size_sampled(orc):
    """Rolling-cache decode workload: batch 64, 32 heads, d=128, w=4096, g=4,
    positions uniform in [4096, 131072]; 64 sampled (batch, head) pairs."""
    dev = _dev()
    B, H, d, w, g = 64, 32, 128, 4096, 4
    q, kc, vc, pos = synth.decode_problem(B, H, d, g + w, w, 131072, torch.bfloat16, seed=4, device=dev)
    rng = np.random.default_rng(4)
    units = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, B, 64), rng.integers(0, H, 64))})
    err = _decode_vs_oracle(orc, q, kc, vc, pos, w, g, 0.0, units=units)
    print(f"decode full size: max-abs {err:.3g} over {len(units)} units")


def test_decode_deterministic():
    dev = _dev()
    q, kc, vc, pos = synth.decode_problem(4, 8, 128, 1028, 1024, 9000, torch.bfloat16, seed=7, device=dev)
    a = swa.decode(q, kc, vc, pos, w=1024, g=4)
    b = swa.decode(q, kc, vc, pos, w=1024, g=4)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_ignores_unwritten_rows(orc, dtype):
    """Ring slots and sink rows never written hold NaN; decode at early
    positions (ring not yet full, sinks still inside the window) stays finite
    and equals the oracle."""
    dev = _dev()
    w, g, d = 64, 4, 128
    positions = [0, 1, 5, 30, 62]
    B, H = len(positions), 2
    n = max(positions) + 1
    kseq = synth.normal((B, H, n, d), seed=35, dtype=dtype, device="cpu")
    vseq = synth.normal((B, H, n, d), seed=36, dtype=dtype, device="cpu")
    q = synth.normal((B, H, d), seed=37, dtype=dtype, device="cpu").to(dev)
    kc = torch.full((B, H, g + w, d), float("nan"), dtype=dtype, device=dev)
    vc = torch.full_like(kc, float("nan"))
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    for b, p in enumerate(positions):
        swa.kv_append(kc[b:b + 1], vc[b:b + 1], kseq[b:b + 1, :, :p + 1].contiguous().to(dev),
                      vseq[b:b + 1, :, :p + 1].contiguous().to(dev), zero, w=w, g=g)
    pos = torch.tensor(positions, dtype=torch.int64, device=dev)
    _decode_vs_oracle(orc, q, kc, vc, pos, w, g, 0.0)


def _one_hot_read_rows(decode_call, B, H, R, d, dtype, dev, fp8_codes=False):
    """Which cache rows a decode reads, read out bit-exactly through the real
    kernel: with q = 0 every attended score is equal (the sink bias is 0), so
    o = mean of the attended V rows; run r sets V[row, c] = [row == r d + c],
    and o[c] != 0 exactly when row r d + c was read (exp(-inf) is 0 and each
    weight 1/|A| is representable and nonzero)."""
    read = np.zeros((B, H, R), dtype=bool)
    for r in range((R + d - 1) // d):
        v = torch.zeros(R, d, dtype=torch.float32)
        for c in range(d):
            if r * d + c < R:
                v[r * d + c, c] = 1.0
        if fp8_codes:
            v = v.to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            v = v.to(dtype)
        o = decode_call(v.to(dev))
        torch.cuda.synchronize()
        nz = (o.float().cpu().numpy() != 0.0)
        lim = min(d, R - r * d)
        read[:, :, r * d:r * d + lim] = nz[:, :, :lim]
    return read


@pytest.mark.parametrize("kind", ["mha_f32", "mha_bf16", "gqa_bf16", "fp8"])
@pytest.mark.parametrize("d,w,g", [(64, 100, 4), (128, 200, 4), (64, 37, 9)])
def test_decode_connectivity_one_hot(kind, d, w, g):
    """The decode kernel's read set over ring and sink rows, bit for bit, at
    the ring and sink edge positions {0, g-1, w-1, w, w+g-1, 3w+7}: ring row
    g + (t mod w) for each window position t <= p, and sink row t for t < g
    only once t has left the window ("Local and Sparse Attention: Reading
    Fewer Token Positions", Figure 2 -- an anchor in the window is read once
    -- and Figure 4 -- the circular overwrite).  The expected rows come from
    the oracle's cache model."""
    dev = _dev()
    positions = sorted({0, g - 1, w - 1, w, w + g - 1, 3 * w + 7} - {-1})
    B, R = len(positions), g + w
    H, Hkv = (4, 1) if kind == "gqa_bf16" else (2, 2)
    dtype = torch.float32 if kind == "mha_f32" else torch.bfloat16
    pos = torch.tensor(positions, dtype=torch.int64, device=dev)
    q = torch.zeros(B, H, d, dtype=dtype, device=dev)
    if kind == "fp8":
        kc = torch.zeros(B, Hkv, R, d, dtype=torch.uint8, device=dev)
        ones = torch.ones(B, Hkv, dtype=torch.float32, device=dev)

        def call(v1):
            vc = v1.expand(B, Hkv, R, d).contiguous()
            return swa.decode_fp8(q, kc, vc, ones, ones, pos, w=w, g=g)
    else:
        kc = torch.zeros(B, Hkv, R, d, dtype=dtype, device=dev)

        def call(v1):
            vc = v1.expand(B, Hkv, R, d).contiguous()
            return swa.decode(q, kc, vc, pos, w=w, g=g)

    read = _one_hot_read_rows(call, B, H, R, d, dtype, dev, fp8_codes=(kind == "fp8"))
    for b, p in enumerate(positions):
        want = np.zeros(R, dtype=bool)
        want[cache_model.logical_rows(p, w, g)[1]] = True
        for h in range(H):
            got = read[b, h]
            assert np.array_equal(got, want), (
                f"{kind} p={p}: rows read {np.flatnonzero(got).tolist()} vs {np.flatnonzero(want).tolist()}")
