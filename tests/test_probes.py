"""The measurement kernels of include/swa_probe.h run through the C ABI:
the MFMA stream leaves a finite checksum per lane equal across identical
launches, and the streaming read of a buffer of ones reads it without
touching the sink (its checksum of 4-word XORs is 0, not the trigger)."""
import pytest
import torch

import block_sparse_causal_band_amd as swa

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_is_deterministic():
    dev = torch.device("cuda")
    wg, iters = 8, 64
    a = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device=dev)
    b = torch.full_like(a, float("nan"))
    print(f"probe_mfma_bf16 workgroups={wg} iters={iters}", flush=True)
    fa = swa.probe_mfma_bf16(a, wg, iters)
    fb = swa.probe_mfma_bf16(b, wg, iters)
    torch.cuda.synchronize()
    assert fa == fb == wg * 4 * iters * 4 * 32768
    assert torch.isfinite(a).all() and torch.equal(a, b)
    assert (a > 0).any()


@pytest.mark.parametrize("streams", [1, 2, 4, 8])
def test_read_probe_runs(streams):
    dev = torch.device("cuda")
    wg = 16
    buf = torch.ones(wg * 32768 * 2 // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(wg, dtype=torch.int32, device=dev)
    print(f"probe_hbm_read bytes={buf.numel() * 4} workgroups={wg} streams={streams}", flush=True)
    assert swa.probe_hbm_read(buf, wg, streams, sink) == buf.numel() * 4
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
