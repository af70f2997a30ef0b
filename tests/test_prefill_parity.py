"""HIP prefill kernel (through the C ABI) against the fp64 oracle.

Tolerances (max-abs over every compared element): fp32 1e-4 and bf16 2e-2,
the contract for this operation.  bf16 sweeps are also held to a normwise
relative error ||o - o_ref||_2 / ||o_ref||_2 below 1e-2, which is tighter
than 2e-2 max-abs when the outputs are small (wide windows average many
values); bf16 rounding of P and of the output alone gives about 2^-9.
The connectivity is checked bit-exactly through a one-hot read-out of the
real kernel.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_causal_band_amd as swa
from block_sparse_causal_band_amd import synth

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2
DEV = "cuda"


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device(DEV)


def _run(q, k, v, w, g, beta=0.0, lse=True):
    out = swa.prefill(q, k, v, w=w, g=g, sink_bias=beta, return_lse=lse)
    torch.cuda.synchronize()
    return out


def _compare(orc, q, k, v, w, g, beta, rows=None, heads=None, tol=None):
    """GPU prefill vs oracle on the given rows (default all) and (b, h) slices."""
    o, lse = _run(q, k, v, w, g, beta)
    B, H, n, d = q.shape
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    if tol is None:
        tol = BF16_TOL if q.dtype == torch.bfloat16 else F32_TOL
    worst, worst_rel, worst_lse = 0.0, 0.0, 0.0
    for b, h in heads:
        qh, kh, vh = (t[b, h].cpu() for t in (q, k, v))
        ro, rl = orc.prefill(qh, kh, vh, w=w, g=g, beta=beta, rows=rows)
        go = o[b, h].float().cpu().numpy()
        gl = lse[b, h].cpu().numpy()
        if rows is not None:
            go, gl = go[rows], gl[rows]
        assert np.all(np.isfinite(go)), "non-finite output"
        err = float(np.max(np.abs(go - ro)))
        worst = max(worst, err)
        worst_rel = max(worst_rel, float(np.linalg.norm(go - ro) / (np.linalg.norm(ro) + 1e-30)))
        worst_lse = max(worst_lse, float(np.max(np.abs(gl - rl))))
    assert worst <= tol, f"max-abs {worst:.3g} > {tol} (n={n}, w={w}, g={g}, {q.dtype})"
    # LSE is fp32 in both paths; its error follows the score error
    assert worst_lse <= (1e-4 if q.dtype == torch.float32 else 2e-2), f"lse max-abs {worst_lse:.3g}"
    return worst, worst_rel


# ---- tiny fp32 workload: batch 1, 1 head, n=256, d=64, w=64, seed 1 ----
def test_tiny_fp32_all_rows(orc):
    dev = _dev()
    q, k, v = synth.qkv(1, 1, 256, 64, torch.float32, seed=1, device="cpu")
    err, _ = _compare(orc, q.to(dev), k.to(dev), v.to(dev), w=64, g=0, beta=0.0)
    print(f"tiny fp32 max-abs {err:.3g}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
def test_fig1_shape(orc, dtype, d):
    """n = 8, w = 3: the worked example's shape, every row."""
    dev = _dev()
    q, k, v = synth.qkv(1, 1, 8, d, dtype, seed=11, device="cpu")
    _compare(orc, q.to(dev), k.to(dev), v.to(dev), w=3, g=0, beta=0.0)


SWEEP = [
    # (B, H, n, d, w, g, beta): several tiles, ragged tails, band/tile edge cases
    (1, 2, 1000, 128, 300, 4, 4.0),
    (2, 1, 777, 64, 64, 0, 0.0),
    (1, 1, 513, 128, 1, 0, 0.0),
    (1, 1, 513, 128, 63, 0, 0.0),
    (1, 1, 513, 64, 65, 1, -1.0),
    (1, 1, 600, 128, 127, 0, 0.0),
    (1, 1, 600, 128, 128, 65, 2.0),
    (1, 1, 600, 64, 129, 130, 0.0),
    (1, 1, 300, 128, 5000, 0, 0.0),   # w > n: full causal attention
    (1, 3, 129, 64, 17, 200, 1.0),    # g > n
    (1, 1, 1, 128, 4, 4, 4.0),        # one token
    (3, 2, 65, 128, 64, 0, 0.0),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,H,n,d,w,g,beta", SWEEP)
def test_sweep(orc, dtype, B, H, n, d, w, g, beta):
    dev = _dev()
    q, k, v = synth.qkv(B, H, n, d, dtype, seed=1000 + n + w + g, device="cpu")
    err, rel = _compare(orc, q.to(dev), k.to(dev), v.to(dev), w=w, g=g, beta=beta)
    if dtype == torch.bfloat16:
        assert rel < 1e-2, f"bf16 normwise relative error {rel:.3g}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_random_shapes(orc, dtype):
    """Seeded random shapes: ragged n, windows narrower and wider than a tile
    or the sequence, sinks, grouped heads, both head sizes, every row."""
    dev = _dev()
    rng = np.random.default_rng(77)
    for case in range(8):
        n = int(rng.integers(1, 700))
        w = int(rng.integers(1, 800))
        g = int(rng.integers(0, 70))
        d = int(rng.choice([64, 128]))
        H, Hkv = [(1, 1), (2, 2), (4, 2), (3, 1)][case % 4]
        beta = float(rng.uniform(-2.0, 4.0))
        q, k, v = synth.qkv(1, H, n, d, dtype, seed=100 + case, kv_heads=Hkv)
        o, lse = _run(q.to(dev), k.to(dev), v.to(dev), w, g, beta)
        tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
        for h in range(H):
            j = h // (H // Hkv)
            ro, rl = orc.prefill(q[0, h], k[0, j], v[0, j], w=w, g=g, beta=beta)
            go = o[0, h].float().cpu().numpy()
            assert np.all(np.isfinite(go))
            err = float(np.max(np.abs(go - ro)))
            assert err <= tol, f"case {case}: n={n} w={w} g={g} d={d} H={H}/{Hkv}: max-abs {err:.3g}"
            assert float(np.max(np.abs(lse[0, h].cpu().numpy() - rl))) <= (1e-4 if dtype == torch.float32 else 2e-2)


def test_full_window_matches_causal_sdpa():
    """w >= n is ordinary causal attention (fp32 torch math on the CPU)."""
    dev = _dev()
    q, k, v = synth.qkv(1, 2, 200, 64, torch.float32, seed=5, device="cpu")
    o = _run(q.to(dev), k.to(dev), v.to(dev), w=200, g=0, lse=False).cpu()
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double(), is_causal=True)
    assert float((o.double() - ref).abs().max()) <= F32_TOL


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,w,g,d", [(8, 3, 0, 64), (8, 3, 1, 64), (256, 64, 0, 64), (300, 70, 4, 128),
                                     (200, 1, 3, 64), (130, 200, 0, 128)])
def test_connectivity_bit_exact(orc, dtype, n, w, g, d):
    """Q = 0 and V[j, c] = [j == r d + c] in run r: O[i, c] != 0 exactly when
    key r d + c is attended by query i.  exp(-inf) = 0 exactly and every
    attended weight is positive, so the nonzero pattern is the kernel's
    connectivity; a zeroed (instead of -inf) score would show up as a nonzero."""
    dev = _dev()
    mask = orc.mask(n, w, g).astype(bool)
    got = np.zeros((n, n), dtype=bool)
    q = torch.zeros(1, 1, n, d, dtype=dtype, device=dev)
    k = synth.normal((1, 1, n, d), seed=3, dtype=dtype, device="cpu").to(dev)
    for r in range((n + d - 1) // d):
        v = torch.zeros(1, 1, n, d, dtype=dtype)
        for c in range(d):
            j = r * d + c
            if j < n:
                v[0, 0, j, c] = 1.0
        o = _run(q, k, v.to(dev), w=w, g=g, lse=False)[0, 0].float().cpu().numpy()
        cols = min(d, n - r * d)
        got[:, r * d:r * d + cols] = o[:, :cols] != 0.0
    assert np.array_equal(got, mask), f"connectivity differs in {int((got != mask).sum())} cells"
    if (n, w, g) == (8, 3, 0):
        assert got.sum() == 21


def test_never_reads_past_n(orc):
    """Rows >= n of the underlying buffers hold NaN; the output stays finite."""
    dev = _dev()
    n, d, pad = 200, 128, 300
    buf = [torch.full((n + pad, d), float("nan"), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    q, k, v = synth.qkv(1, 1, n, d, torch.bfloat16, seed=9, device="cpu")
    for b, t in zip(buf, (q, k, v)):
        b[:n] = t[0, 0].to(dev)
    views = [b[:n].view(1, 1, n, d) for b in buf]
    o, lse = _run(*views, w=50, g=2, beta=1.0)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    ro, _ = orc.prefill(q[0, 0], k[0, 0], v[0, 0], w=50, g=2, beta=1.0)
    assert float(np.max(np.abs(o[0, 0].float().cpu().numpy() - ro))) <= BF16_TOL


@pytest.mark.parametrize("case", ["ramp", "spikes"])
def test_reference_max_moves_inside_full_tiles(orc, case):
    """Scores that keep rising along the sequence (keys scaled up with their
    position), or single keys whose scores jump far past everything before
    them (some past the fp32 range of 2^x against the old reference), make the
    running reference max move inside runs of FULL tiles, where the kernel
    forms the probabilities before it knows the tile's row max."""
    dev = _dev()
    B, H, n, d, w, g = 1, 2, 1500, 128, 300, 2
    q, k, v = synth.qkv(B, H, n, d, torch.bfloat16, seed=31, device="cpu")
    if case == "ramp":
        k = (k.float() * torch.linspace(0.3, 3.0, n).view(1, 1, n, 1)).to(torch.bfloat16)
    else:
        kf = k.float()
        for j, a in ((400, 12.0), (700, 40.0), (701, -40.0), (1000, 80.0), (1333, 25.0)):
            kf[:, :, j] *= a
        k = kf.to(torch.bfloat16)
    _compare(orc, q.to(dev), k.to(dev), v.to(dev), w, g, 1.0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_more_sinks_than_positions_is_g_equal_n(dtype):
    """g past n (up to INT_MAX) selects every position as a sink, as g = n
    does: the same output bit for bit, for the plain and the landmark
    prefill (the tile arithmetic on g stays within int)."""
    dev = _dev()
    n = 300
    q, k, v = synth.qkv(1, 2, n, 128, dtype, seed=31, device=dev)
    ref, lref = swa.prefill(q, k, v, w=40, g=n, sink_bias=1.5, return_lse=True)
    for g in (n + 5, 2 ** 31 - 1):
        print(f"prefill {dtype} n={n} g={g}", flush=True)
        o, lo = swa.prefill(q, k, v, w=40, g=g, sink_bias=1.5, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, ref) and torch.equal(lo, lref), g
    lm_ref, lm_lref = swa.landmark_prefill(q, k, v, w=40, g=n, r=16, sink_bias=1.5, return_lse=True)
    lm, lm_l = swa.landmark_prefill(q, k, v, w=40, g=2 ** 31 - 1, r=16, sink_bias=1.5, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(lm, lm_ref) and torch.equal(lm_l, lm_lref)


def test_deterministic():
    dev = _dev()
    q, k, v = synth.qkv(1, 4, 3000, 128, torch.bfloat16, seed=21, device=dev)
    a = _run(q, k, v, w=1000, g=4, beta=4.0)
    b = _run(q, k, v, w=1000, g=4, beta=4.0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _sample_rows(n, w, count, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 63, 64, 127, 128, w - 2, w - 1, w, w + 1, w + 127, n - 129, n - 128, n - 2, n - 1]
    rest = rng.choice(n, size=count, replace=False).tolist()
    return sorted({r for r in fixed + rest if 0 <= r < n})


# Full-size workloads, sampled rows of a few heads.
FULL = [
    # name, B, H, n, d, w, g, beta, seed
    ("mistral_prefill", 1, 32, 16384, 128, 4096, 0, 0.0, 2),
    ("sink_prefill", 1, 32, 32768, 128, 4096, 4, 4.0, 3),
    ("gemma3_local_prefill", 1, 16, 131072, 128, 1024, 0, 0.0, 5),
]


@pytest.mark.parametrize("name,B,H,n,d,w,g,beta,seed", FULL)
def test_full_size_sampled_rows(orc, name, B, H, n, d, w, g, beta, seed):
    dev = _dev()
    q, k, v = synth.qkv(B, H, n, d, torch.bfloat16, seed=seed, device=dev)
    rows = _sample_rows(n, w, 48, seed)
    heads = [(0, 0), (0, H // 2), (0, H - 1)]
    err, rel = _compare(orc, q, k, v, w=w, g=g, beta=beta, rows=rows, heads=heads)
    print(f"{name}: max-abs {err:.3g}, normwise relative {rel:.3g} over {len(rows)} rows x {len(heads)} heads")
    assert rel < 1e-2
