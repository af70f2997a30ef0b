"""The three calls of the boundary -- swa_prefill_fwd, swa_kv_append and
swa_decode_fwd -- called directly through ctypes (no binding wrapper) on
valid problems, against the oracle (prefill, decode) and the cache model
(append, bit for bit)."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_causal_band_amd as swa
from block_sparse_causal_band_amd import synth
from oracle import cache_model
from tests.parity import gate

pytestmark = pytest.mark.gpu


def _code(dtype):
    return swa.SWA_BF16 if dtype == torch.bfloat16 else swa.SWA_F32


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
def test_swa_prefill_fwd_direct(orc, dtype, d):
    dev = torch.device("cuda")
    B, H, n, w, g, beta = 2, 3, 300, 70, 4, 2.0
    q, k, v = synth.qkv(B, H, n, d, dtype, seed=201)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, n), float("nan"), dtype=torch.float32, device=dev)
    print(f"swa_prefill_fwd {dtype} d={d} n={n} w={w} g={g}", flush=True)
    rc = swa.lib().swa_prefill_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                                   n, d, w, g, ctypes.c_float(d ** -0.5), ctypes.c_float(beta), _code(dtype),
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == 0, swa.strerror(rc)
    torch.cuda.synchronize()
    for b in range(B):
        ro, rl = orc.prefill(q[b], k[b], v[b], w=w, g=g, beta=beta)
        gate(o[b].float().cpu().numpy(), ro, dtype, f"swa_prefill_fwd b={b}")
        gate(lse[b].cpu().numpy(), rl, dtype, "swa_prefill_fwd lse")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_swa_kv_append_and_decode_fwd_direct(orc, dtype):
    """Append a prefix 0..p-1 in one call and token p in a second, then decode
    at p, each through its C name; then decode over a split launch (few
    (batch, head) pairs) with a caller workspace."""
    dev = torch.device("cuda")
    d, w, g, beta = 128, 96, 4, 1.0
    positions = [0, 3, 95, 96, 99, 300]
    B, H = len(positions), 2
    L = swa.lib()
    stream = torch.cuda.current_stream().cuda_stream
    n = max(positions) + 1
    kseq = synth.normal((B, H, n, d), seed=202, dtype=dtype)
    vseq = synth.normal((B, H, n, d), seed=203, dtype=dtype)
    q = synth.normal((B, H, d), seed=204, dtype=dtype)
    kc = torch.zeros(B, H, g + w, d, dtype=dtype, device=dev)
    vc = torch.zeros_like(kc)
    ref_k = torch.zeros(B, H, g + w, d, dtype=dtype)
    ref_v = torch.zeros_like(ref_k)
    for b, p in enumerate(positions):
        for start, stop in ((0, p), (p, p + 1)):
            if stop <= start:
                continue
            kn = kseq[b:b + 1, :, start:stop].contiguous()
            vn = vseq[b:b + 1, :, start:stop].contiguous()
            knd, vnd = kn.to(dev), vn.to(dev)
            pos0 = torch.tensor([start], dtype=torch.int64, device=dev)
            rc = L.swa_kv_append(kc[b:b + 1].data_ptr(), vc[b:b + 1].data_ptr(), knd.data_ptr(), vnd.data_ptr(),
                                 pos0.data_ptr(), 1, H, stop - start, d, w, g, _code(dtype), stream)
            assert rc == 0, swa.strerror(rc)
            torch.cuda.synchronize()
            cache_model.append(ref_k[b:b + 1], ref_v[b:b + 1], kn, vn, [start], w, g)
    assert torch.equal(kc.cpu(), ref_k) and torch.equal(vc.cpu(), ref_v), "swa_kv_append vs the cache model"

    qd = q.to(dev)
    pos = torch.tensor(positions, dtype=torch.int64, device=dev)
    need = int(L.swa_decode_workspace_bytes(B, H, d, w, g))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=dev)
    print(f"swa_decode_fwd {dtype} B={B} H={H} w={w} g={g} workspace {need} B", flush=True)
    rc = L.swa_decode_fwd(qd.data_ptr(), kc.data_ptr(), vc.data_ptr(), pos.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          B, H, d, w, g, ctypes.c_float(d ** -0.5), ctypes.c_float(beta), _code(dtype),
                          ws.data_ptr() if need else None, need, stream)
    assert rc == 0, swa.strerror(rc)
    torch.cuda.synchronize()
    for b, p in enumerate(positions):
        qseq = torch.zeros(H, p + 1, d, dtype=torch.float64)
        qseq[:, p] = q[b].double()
        ro, rl = orc.prefill(qseq, kseq[b, :, :p + 1], vseq[b, :, :p + 1], w=w, g=g, beta=beta, rows=[p])
        gate(o[b].float().cpu().numpy(), ro[:, 0], dtype, f"swa_decode_fwd p={p}")
        gate(lse[b].cpu().numpy(), rl[:, 0], dtype, "swa_decode_fwd lse")
