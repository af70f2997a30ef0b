"""Exact causal sliding-window attention with attention sinks for AMD MI355X.

The computation lives in libswa.so (hand-written HIP kernels for gfx950
behind the C ABI of include/swa.h, with the measurement kernels of
include/swa_probe.h); this package is its thin Python binding.

    from block_sparse_causal_band_amd import prefill, kv_append, decode
    from block_sparse_causal_band_amd import chunk_prefill, lse_merge
    from block_sparse_causal_band_amd import kv_append_fp8, decode_fp8
    from block_sparse_causal_band_amd import decode_noalloc
    from block_sparse_causal_band_amd import dilated_prefill, landmark_prefill

Importing the package does not load the library; the first call does, and
raises if it is not built (``python -m block_sparse_causal_band_amd.build``).
"""
from .binding import (  # noqa: F401
    SWA_BF16,
    SWA_F32,
    SwaError,
    band_tiles,
    chunk_prefill,
    decode,
    decode_fp8,
    decode_noalloc,
    decode_scratch_bytes,
    decode_workspace_bytes,
    dilated_prefill,
    kv_append,
    kv_append_fp8,
    landmark_prefill,
    landmark_workspace_bytes,
    lib,
    lse_merge,
    prefill,
    prefill_order,
    prefill_tile_shape,
    probe_hbm_read,
    probe_mfma_bf16,
    strerror,
)
