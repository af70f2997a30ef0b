"""The decode entry point that allocates nothing (swa_decode_fwd_gqa_noalloc)
against the workspace form (swa_decode_fwd_gqa), both called through the C
ABI on the same inputs.  The two share their kernels, so the outputs and
LSEs must agree bit for bit.  Each case makes two calls in a row, the second
on a smaller problem, and every shape here splits the cache rows across
workgroups, so the fixed scratch really holds the partial results (and the
second call must not see the first call's leftovers)."""
import ctypes

import pytest
import torch

import block_sparse_causal_band_amd as swa
from block_sparse_causal_band_amd import synth

pytestmark = pytest.mark.gpu


def _dtype_code(dt):
    return swa.SWA_BF16 if dt == torch.bfloat16 else swa.SWA_F32


def _problem(B, H, Hkv, d, w, g, dtype, seed):
    dev = torch.device("cuda")
    q, kc, vc, pos = synth.decode_problem(B, H, d, g + w, 0, 3 * w + 7, dtype, seed=seed, device=dev, kv_heads=Hkv)
    return q, kc, vc, pos


def _both(B, H, Hkv, d, w, g, dtype, seed, beta):
    L = swa.lib()
    q, kc, vc, pos = _problem(B, H, Hkv, d, w, g, dtype, seed)
    stream = torch.cuda.current_stream().cuda_stream
    scale = d ** -0.5
    need = int(L.swa_decode_workspace_bytes_gqa(B, H, Hkv, d, w, g))
    assert need > 0, "the case must split (otherwise the scratch is not used)"
    assert need <= int(L.swa_decode_scratch_bytes())
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    o_ref = torch.full_like(q, float("nan"))
    l_ref = torch.full((B, H), float("nan"), dtype=torch.float32, device=q.device)
    rc = L.swa_decode_fwd_gqa(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), pos.data_ptr(), o_ref.data_ptr(),
                              l_ref.data_ptr(), B, H, Hkv, d, w, g, ctypes.c_float(scale), ctypes.c_float(beta),
                              _dtype_code(dtype), ws.data_ptr(), need, stream)
    assert rc == 0, swa.strerror(rc)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=q.device)
    rc = L.swa_decode_fwd_gqa_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), pos.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), B, H, Hkv, d, w, g, ctypes.c_float(scale),
                                      ctypes.c_float(beta), _dtype_code(dtype), stream)
    assert rc == 0, swa.strerror(rc)
    torch.cuda.synchronize()
    assert torch.isfinite(o_ref.float()).all() and torch.isfinite(l_ref).all()
    assert torch.equal(o.view(torch.int16) if dtype == torch.bfloat16 else o.view(torch.int32),
                       o_ref.view(torch.int16) if dtype == torch.bfloat16 else o_ref.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("first,second", [
    # (B, H, Hkv, d, w, g): multi-head (the vector kernel), split 16 ways, then 4 ways
    ((2, 8, 8, 128, 4096, 4), (1, 4, 4, 128, 1024, 0)),
    # grouped query heads (bf16: the matrix-core kernel), then a smaller group
    ((2, 16, 4, 128, 2048, 4), (1, 4, 2, 64, 512, 2)),
])
def test_noalloc_matches_workspace_form(dtype, first, second):
    print(f"noalloc decode {dtype} {first} then {second}", flush=True)
    _both(*first, dtype, seed=11, beta=1.5)
    _both(*second, dtype, seed=12, beta=0.0)
