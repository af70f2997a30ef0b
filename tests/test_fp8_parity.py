"""FP8 (E4M3) window KV cache on the HIP path (through the C ABI) against
the oracle.

kv_append_fp8 must store exactly the oracle's codes (byte work: bit-exact),
quantised from the same inputs with the same per-(batch, head) scales and
written where the token-by-token cache model puts them.  decode_fp8 is
compared with the oracle's decode over the dequantised rows (scale x code
value, exact in fp64): fp32 q 1e-4, bf16 q 2e-2 max-abs.
"""
import numpy as np
import pytest
import torch

import block_sparse_causal_band_amd as swa
import oracle
from block_sparse_causal_band_amd import synth
from oracle import cache_model, fp8
from tests.parity import gate

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda")


def _tol(dtype):
    return 2e-2 if dtype == torch.bfloat16 else 1e-4


def _wide_values(shape, seed, dtype):
    """N(0,1) times 10^U(-4, 3): subnormal codes, saturation and everything between."""
    x = synth.normal(shape, seed=seed, dtype=torch.float32)
    mag = synth.normal(shape, seed=seed + 100, dtype=torch.float32).clamp(-2, 2) * 1.75 - 0.5
    return (x * torch.pow(10.0, mag)).to(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w,g,T,starts", [(8, 4, 3, [0, 2, 40]), (8, 0, 13, [0, 1, 9]), (5, 3, 30, [0, 2, 7]),
                                          (64, 4, 64, [0, 64, 1000])])
def test_fp8_append_bit_exact(dtype, d, w, g, T, starts):
    dev = _dev()
    B, H = len(starts), 2
    kn = _wide_values((B, H, T, d), 81, dtype)
    vn = _wide_values((B, H, T, d), 82, dtype)
    kn[0, 0, 0, :4] = torch.tensor([float("inf"), -float("inf"), 0.0, -0.0], dtype=dtype)
    ks = torch.rand(B, H, generator=torch.Generator().manual_seed(83)) * 2 + 0.01
    vs = torch.rand(B, H, generator=torch.Generator().manual_seed(84)) * 2 + 0.01
    pos = torch.tensor(starts, dtype=torch.int64)
    init = torch.full((B, H, g + w, d), 0x55, dtype=torch.uint8)
    ref_k, ref_v = init.clone().numpy(), init.clone().numpy()
    qk = fp8.quantize(kn.float().numpy(), ks.numpy()[:, :, None, None])
    qv = fp8.quantize(vn.float().numpy(), vs.numpy()[:, :, None, None])
    cache_model.append(ref_k, ref_v, qk, qv, pos.tolist(), w, g)
    gk, gv = init.to(dev), init.to(dev)
    swa.kv_append_fp8(gk, gv, kn.to(dev), vn.to(dev), pos.to(dev), ks.to(dev), vs.to(dev), w=w, g=g)
    torch.cuda.synchronize()
    bad_k = np.nonzero(gk.cpu().numpy() != ref_k)
    assert bad_k[0].size == 0, f"{bad_k[0].size} K bytes differ"
    assert np.array_equal(gv.cpu().numpy(), ref_v)


def test_fp8_append_nan_gives_nan_code():
    dev = _dev()
    kn = torch.zeros(1, 1, 1, 64, dtype=torch.float32)
    kn[0, 0, 0, 0] = float("nan")
    kc = torch.zeros(1, 1, 8, 64, dtype=torch.uint8, device=dev)
    one = torch.ones(1, 1, dtype=torch.float32, device=dev)
    swa.kv_append_fp8(kc, kc.clone(), kn.to(dev), kn.to(dev), torch.zeros(1, dtype=torch.int64, device=dev), one,
                      one, w=8, g=0)
    torch.cuda.synchronize()
    assert int(kc[0, 0, 0, 0]) & 0x7F == 0x7F


def _decode_fp8_vs_oracle(orc, q, kc, vc, ks, vs, pos, w, g, beta, units=None):
    B, H, d = q.shape
    Hkv = kc.shape[1]
    o, lse = swa.decode_fp8(q, kc, vc, ks, vs, pos, w=w, g=g, sink_bias=beta, return_lse=True)
    torch.cuda.synchronize()
    if units is None:
        units = [(b, h) for b in range(B) for h in range(H)]
    pos_h = pos.cpu().tolist()
    ks_h, vs_h = ks.cpu().double().numpy(), vs.cpu().double().numpy()
    nk = g + w
    qs, ps, kps, kk_l, vv_l = [], [], [], [], []
    for b, h in units:
        p = pos_h[b]
        j = oracle.kv_head_of(h, H, Hkv)
        positions, rows = cache_model.logical_rows(p, w, g)
        kp = np.full(nk, -1, dtype=np.int64)
        kp[:len(positions)] = positions
        rows_t = torch.as_tensor(rows, device=kc.device)
        kk = np.zeros((nk, d))
        vv = np.zeros((nk, d))
        kk[:len(rows)] = ks_h[b, j] * fp8.decode(kc[b, j].index_select(0, rows_t).cpu().numpy())
        vv[:len(rows)] = vs_h[b, j] * fp8.decode(vc[b, j].index_select(0, rows_t).cpu().numpy())
        qs.append(q[b, h].double().cpu().numpy()); ps.append(p); kps.append(kp); kk_l.append(kk); vv_l.append(vv)
    ro, rl = orc.decode(np.stack(qs), ps, np.stack(kps), np.stack(kk_l), np.stack(vv_l), w=w, g=g, beta=beta)
    go = torch.stack([o[b, h] for b, h in units]).float().cpu().numpy()
    gl = torch.stack([lse[b, h] for b, h in units]).cpu().numpy()
    err, _ = gate(go, ro, q.dtype, f"fp8 decode H={H} Hkv={Hkv} w={w} g={g}")
    gate(gl, rl, q.dtype, "fp8 decode lse")
    return err


EDGE_POS = lambda w, g: sorted({0, 1, 2, 3, g, w - 2, w - 1, w, w + 1, w + 2, w + g - 1, w + g, 3 * w + 7})


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("w,g,beta", [(16, 0, 0.0), (16, 4, 0.0), (100, 4, 4.0), (7, 9, -1.0)])
def test_fp8_decode_through_appended_cache(orc, dtype, d, w, g, beta):
    """Fill fp8 caches by kv_append_fp8 with positions 0..p, decode at p."""
    dev = _dev()
    positions = [p for p in EDGE_POS(w, g) if p >= 0]
    B, H = len(positions), 2
    n = max(positions) + 1
    kseq = synth.normal((B, H, n, d), seed=85, dtype=dtype, device="cpu")
    vseq = synth.normal((B, H, n, d), seed=86, dtype=dtype, device="cpu")
    q = synth.normal((B, H, d), seed=87, dtype=dtype, device="cpu").to(dev)
    ks = (torch.rand(B, H, generator=torch.Generator().manual_seed(88)) * 0.05 + 0.01).to(dev)
    vs = (torch.rand(B, H, generator=torch.Generator().manual_seed(89)) * 0.05 + 0.01).to(dev)
    kc = torch.full((B, H, g + w, d), 0x7F, dtype=torch.uint8, device=dev)  # NaN codes: unwritten rows must not be read
    vc = kc.clone()
    for b, p in enumerate(positions):
        one = torch.zeros(1, dtype=torch.int64, device=dev)
        swa.kv_append_fp8(kc[b:b + 1], vc[b:b + 1], kseq[b:b + 1, :, :p + 1].contiguous().to(dev),
                          vseq[b:b + 1, :, :p + 1].contiguous().to(dev), one, ks[b:b + 1], vs[b:b + 1], w=w, g=g)
    pos = torch.tensor(positions, dtype=torch.int64, device=dev)
    _decode_fp8_vs_oracle(orc, q, kc, vc, ks, vs, pos, w, g, beta)


@pytest.mark.parametrize("q_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,H,Hkv", [(1, 1, 1), (2, 8, 2), (3, 16, 2), (8, 64, 64)])
def test_fp8_decode_split_gqa(orc, q_dtype, B, H, Hkv):
    """Split and unsplit launches, one to eight query heads per workgroup."""
    dev = _dev()
    w, g, d = 700, 4, 128
    q, kc, vc, ks, vs, pos = synth.fp8_decode_problem(B, H, Hkv, d, g + w, w, 5 * w, q_dtype, seed=90, device=dev)
    units = [(b, h) for b in range(B) for h in range(H)][:64]
    _decode_fp8_vs_oracle(orc, q, kc, vc, ks, vs, pos, w, g, 0.5, units=units)


def test_fp8_decode_full_size_sampled(orc):
    """FP8 rolling-cache decode: batch 64, 32 heads, d=128, w=4096, g=4,
    positions uniform in [4096, 131072]; 48 sampled (batch, head) pairs."""
    dev = _dev()
    B, H, d, w, g = 64, 32, 128, 4096, 4
    q, kc, vc, ks, vs, pos = synth.fp8_decode_problem(B, H, H, d, g + w, w, 131072, torch.bfloat16, seed=91,
                                                      device=dev)
    rng = np.random.default_rng(91)
    units = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, B, 48), rng.integers(0, H, 48))})
    _decode_fp8_vs_oracle(orc, q, kc, vc, ks, vs, pos, w, g, 0.0, units=units)


def test_fp8_decode_negative_position_gives_nan():
    dev = _dev()
    q, kc, vc, ks, vs, _ = synth.fp8_decode_problem(2, 4, 2, 128, 20, 0, 0, torch.bfloat16, seed=92, device=dev)
    pos = torch.tensor([-5, 40], dtype=torch.int64, device=dev)
    o = swa.decode_fp8(q, kc, vc, ks, vs, pos, w=16, g=4)
    torch.cuda.synchronize()
    assert torch.isnan(o[0].float()).all() and torch.isfinite(o[1].float()).all()
