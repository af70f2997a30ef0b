"""Python binding of libswa.so (include/swa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Tensors are torch tensors on a ROCm device; the
binding checks their shapes, dtypes and layout, passes raw device pointers,
and enqueues on torch's current stream of the tensors' device.  There is no
fallback: if libswa.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libswa.so")

SWA_F32 = 0
SWA_BF16 = 1

_vp = ctypes.c_void_p
_int = ctypes.c_int
_flt = ctypes.c_float


class SwaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({strerror(status)})")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libswa.so (built in-tree by ``python -m block_sparse_causal_band_amd.build``)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m block_sparse_causal_band_amd.build` "
                "(there is no fallback implementation)"
            )
        L = ctypes.CDLL(LIB_PATH)
        L.swa_prefill_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _int,
                                      _flt, _flt, _int, _vp]
        L.swa_prefill_fwd.restype = _int
        L.swa_kv_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _int, _int, _vp]
        L.swa_kv_append.restype = _int
        L.swa_decode_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int,
                                     _flt, _flt, _int, _vp, ctypes.c_size_t, _vp]
        L.swa_decode_fwd.restype = _int
        L.swa_decode_workspace_bytes.argtypes = [_int] * 5
        L.swa_decode_workspace_bytes.restype = ctypes.c_size_t
        L.swa_prefill_fwd_gqa.argtypes = [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _int, _int,
                                          _flt, _flt, _int, _vp]
        L.swa_prefill_fwd_gqa.restype = _int
        L.swa_decode_fwd_gqa.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _int,
                                         _flt, _flt, _int, _vp, ctypes.c_size_t, _vp]
        L.swa_decode_fwd_gqa.restype = _int
        L.swa_decode_workspace_bytes_gqa.argtypes = [_int] * 6
        L.swa_decode_workspace_bytes_gqa.restype = ctypes.c_size_t
        L.swa_decode_fwd_gqa_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int,
                                                 _int, _flt, _flt, _int, _vp]
        L.swa_decode_fwd_gqa_noalloc.restype = _int
        L.swa_decode_scratch_bytes.argtypes = []
        L.swa_decode_scratch_bytes.restype = ctypes.c_size_t
        L.swa_chunk_prefill_fwd.argtypes = [_vp] * 8 + [_int] * 7 + [ctypes.c_float] * 2 + [_int, _int, _vp]
        L.swa_chunk_prefill_fwd.restype = _int
        L.swa_kv_append_fp8.argtypes = [_vp] * 7 + [_int] * 6 + [_int, _vp]
        L.swa_kv_append_fp8.restype = _int
        L.swa_decode_fwd_fp8.argtypes = ([_vp] * 8 + [_int] * 6 + [ctypes.c_float] * 2 + [_int, _vp, ctypes.c_size_t,
                                                                                           _vp])
        L.swa_decode_fwd_fp8.restype = _int
        L.swa_dilated_prefill_fwd.argtypes = [_vp] * 5 + [_int] * 7 + [ctypes.c_float, _int, _vp]
        L.swa_dilated_prefill_fwd.restype = _int
        L.swa_landmark_prefill_fwd.argtypes = ([_vp] * 5 + [_int] * 8 + [ctypes.c_float] * 2 +
                                               [_int, _vp, ctypes.c_size_t, _vp])
        L.swa_landmark_prefill_fwd.restype = _int
        L.swa_landmark_workspace_bytes.argtypes = [_int] * 5
        L.swa_landmark_workspace_bytes.restype = ctypes.c_size_t
        L.swa_lse_merge.argtypes = [_vp] * 6 + [ctypes.c_longlong, _int, _int, _vp]
        L.swa_lse_merge.restype = _int
        L.swa_strerror.argtypes = [_int]
        L.swa_strerror.restype = ctypes.c_char_p
        L.swa_band_tiles.argtypes = [_int, _int, _int, _int, _int, _vp, ctypes.c_long]
        L.swa_band_tiles.restype = ctypes.c_long
        L.swa_prefill_tile_shape.argtypes = [_int, _int, ctypes.POINTER(_int), ctypes.POINTER(_int)]
        L.swa_prefill_tile_shape.restype = _int
        L.swa_prefill_order.argtypes = [_int, _int, _int, _vp, ctypes.c_long]
        L.swa_prefill_order.restype = ctypes.c_long
        L.swa_probe_mfma_bf16.argtypes = [_vp, _int, _int, _vp]
        L.swa_probe_mfma_bf16.restype = _int
        L.swa_probe_mfma_bf16_flops.argtypes = [_int, _int]
        L.swa_probe_mfma_bf16_flops.restype = ctypes.c_double
        L.swa_probe_hbm_read.argtypes = [_vp, ctypes.c_size_t, _int, _int, _vp, _vp]
        L.swa_probe_hbm_read.restype = _int
        _LIB = L
    return _LIB


def strerror(status: int) -> str:
    return lib().swa_strerror(int(status)).decode()


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype == torch.float32:
        return SWA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream(t) -> int:
    import torch

    return torch.cuda.current_stream(t.device).cuda_stream


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev_tensor(t, name):
    import torch

    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _need(t.is_cuda, f"{name} must be on a ROCm device")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def prefill(q, k, v, w: int, g: int = 0, scale: float | None = None, sink_bias: float = 0.0,
            return_lse: bool = False, out=None):
    """Causal sliding-window attention with sinks: q [batch, heads, n, d] against
    k, v [batch, kv_heads, n, d] (kv_heads == heads: multi-head attention; a
    divisor of heads: grouped-query attention, query head h reads key/value
    head h // (heads // kv_heads))."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name)
    _need(q.dim() == 4 and k.dim() == 4 and k.shape == v.shape, "q, k, v must be 4-d, k and v one shape")
    _need(q.shape[0] == k.shape[0] and q.shape[2:] == k.shape[2:],
          "q [batch, heads, n, d] and k, v [batch, kv_heads, n, d] must agree on batch, n, d")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share one dtype")
    _need(q.device == k.device == v.device, "q, k, v must be on one device")
    B, H, n, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    _dev_tensor(o, "out")
    _need(o.shape == q.shape and o.dtype == q.dtype and o.device == q.device, "out must match q")
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device) if return_lse else None
    rc = lib().swa_prefill_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr() if lse is not None else None,
                                   B, H, Hkv, n, d, int(w), int(g), float(scale), float(sink_bias),
                                   _dtype_code(q), _stream(q))
    if rc != 0:
        raise SwaError(rc, "swa_prefill_fwd_gqa")
    return (o, lse) if return_lse else o


def kv_append(k_cache, v_cache, k_new, v_new, pos, w: int, g: int = 0):
    """Write k_new, v_new [batch, heads, t, d] at positions pos[b] .. pos[b]+t-1."""
    import torch

    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new), ("pos", pos)):
        _dev_tensor(t, name)
    B, H, R, d = k_cache.shape
    _need(v_cache.shape == k_cache.shape, "k_cache and v_cache must share one shape")
    _need(R == g + w, f"cache must hold g + w = {g + w} rows per (batch, head)")
    _need(k_new.dim() == 4 and k_new.shape[:2] == (B, H) and k_new.shape[3] == d, "k_new must be [batch, heads, t, d]")
    _need(v_new.shape == k_new.shape, "v_new must match k_new")
    _need(len({k_cache.dtype, v_cache.dtype, k_new.dtype, v_new.dtype}) == 1, "one dtype for cache and new tokens")
    _need(pos.dtype == torch.int64 and pos.shape == (B,), "pos must be int64 [batch]")
    rc = lib().swa_kv_append(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                             pos.data_ptr(), B, H, k_new.shape[2], d, int(w), int(g),
                             _dtype_code(k_cache), _stream(k_cache))
    if rc != 0:
        raise SwaError(rc, "swa_kv_append")


def _fp8_scales(k_scale, v_scale, B, H):
    import torch

    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _dev_tensor(t, name)
        _need(t.dtype == torch.float32 and t.shape == (B, H), f"{name} must be fp32 [batch, kv_heads]")


def kv_append_fp8(k_cache, v_cache, k_new, v_new, pos, k_scale, v_scale, w: int, g: int = 0):
    """Quantise k_new, v_new [batch, heads, t, d] (bf16 or fp32) to E4M3 codes
    (uint8 caches [batch, heads, g + w, d]) with per-(batch, head) fp32 scales
    [batch, heads], at positions pos[b] .. pos[b]+t-1."""
    import torch

    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new), ("pos", pos)):
        _dev_tensor(t, name)
    _need(k_cache.dtype == v_cache.dtype == torch.uint8, "fp8 caches are uint8 tensors of E4M3 codes")
    B, H, R, d = k_cache.shape
    _need(v_cache.shape == k_cache.shape, "k_cache and v_cache must share one shape")
    _need(R == g + w, f"cache must hold g + w = {g + w} rows per (batch, head)")
    _need(k_new.dim() == 4 and k_new.shape[:2] == (B, H) and k_new.shape[3] == d, "k_new must be [batch, heads, t, d]")
    _need(v_new.shape == k_new.shape and v_new.dtype == k_new.dtype, "v_new must match k_new")
    _need(pos.dtype == torch.int64 and pos.shape == (B,), "pos must be int64 [batch]")
    _fp8_scales(k_scale, v_scale, B, H)
    rc = lib().swa_kv_append_fp8(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                 pos.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), B, H, k_new.shape[2], d,
                                 int(w), int(g), _dtype_code(k_new), _stream(k_cache))
    if rc != 0:
        raise SwaError(rc, "swa_kv_append_fp8")


def decode_fp8(q, k_cache, v_cache, k_scale, v_scale, pos, w: int, g: int = 0, scale: float | None = None,
               sink_bias: float = 0.0, return_lse: bool = False, workspace=None, out=None):
    """decode() over E4M3 caches (uint8 [batch, kv_heads, g + w, d]) with fp32
    scales [batch, kv_heads]; q and the output bf16 or fp32."""
    import torch

    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("pos", pos)):
        _dev_tensor(t, name)
    B, H, d = q.shape
    _need(k_cache.dim() == 4 and k_cache.dtype == v_cache.dtype == torch.uint8, "fp8 caches are uint8 [b, hkv, r, d]")
    Hkv = k_cache.shape[1]
    _need(k_cache.shape == v_cache.shape == (B, Hkv, g + w, d), "caches must be [batch, kv_heads, g + w, d]")
    _need(pos.dtype == torch.int64 and pos.shape == (B,), "pos must be int64 [batch]")
    _fp8_scales(k_scale, v_scale, B, Hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    _dev_tensor(o, "out")
    _need(o.shape == q.shape and o.dtype == q.dtype, "out must match q")
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if return_lse else None
    need = decode_workspace_bytes(B, H, d, w, g, kv_heads=Hkv)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().swa_decode_fwd_fp8(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(),
                                  v_scale.data_ptr(), pos.data_ptr(), o.data_ptr(),
                                  lse.data_ptr() if lse is not None else None, B, H, Hkv, d, int(w), int(g),
                                  float(scale), float(sink_bias), _dtype_code(q), ws_ptr, ws_bytes, _stream(q))
    if rc != 0:
        raise SwaError(rc, "swa_decode_fwd_fp8")
    return (o, lse) if return_lse else o


def decode_workspace_bytes(batch: int, heads: int, d: int, w: int, g: int, kv_heads: int | None = None) -> int:
    if kv_heads is None:
        return int(lib().swa_decode_workspace_bytes(batch, heads, d, w, g))
    return int(lib().swa_decode_workspace_bytes_gqa(batch, heads, kv_heads, d, w, g))


def decode(q, k_cache, v_cache, pos, w: int, g: int = 0, scale: float | None = None, sink_bias: float = 0.0,
           return_lse: bool = False, workspace=None, out=None):
    """One query per (batch, head), q [batch, heads, d], at positions pos [batch],
    against caches [batch, kv_heads, g + w, d] (kv_heads divides heads)."""
    import torch

    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("pos", pos)):
        _dev_tensor(t, name)
    B, H, d = q.shape
    _need(k_cache.dim() == 4, "caches must be [batch, kv_heads, g + w, d]")
    Hkv = k_cache.shape[1]
    _need(k_cache.shape == v_cache.shape == (B, Hkv, g + w, d), f"caches must be [batch, kv_heads, g + w, d]")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "one dtype for q and the caches")
    _need(pos.dtype == torch.int64 and pos.shape == (B,), "pos must be int64 [batch]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    _dev_tensor(o, "out")
    _need(o.shape == q.shape and o.dtype == q.dtype, "out must match q")
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if return_lse else None
    need = decode_workspace_bytes(B, H, d, w, g, kv_heads=Hkv)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().swa_decode_fwd_gqa(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), pos.data_ptr(),
                                  o.data_ptr(), lse.data_ptr() if lse is not None else None, B, H, Hkv, d,
                                  int(w), int(g), float(scale), float(sink_bias), _dtype_code(q), ws_ptr, ws_bytes,
                                  _stream(q))
    if rc != 0:
        raise SwaError(rc, "swa_decode_fwd_gqa")
    return (o, lse) if return_lse else o


def decode_noalloc(q, k_cache, v_cache, pos, w: int, g: int = 0, scale: float | None = None,
                   sink_bias: float = 0.0, lse=None, out=None):
    """decode() through the entry point that allocates nothing: `out` (and
    `lse`, fp32 [batch, heads], if given) must be passed in, and a split
    launch keeps its partial results in the library's fixed device scratch
    (calls that overlap in time on one device race on it)."""
    import torch

    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("pos", pos), ("out", out)):
        _dev_tensor(t, name)
    B, H, d = q.shape
    _need(k_cache.dim() == 4, "caches must be [batch, kv_heads, g + w, d]")
    Hkv = k_cache.shape[1]
    _need(k_cache.shape == v_cache.shape == (B, Hkv, g + w, d), "caches must be [batch, kv_heads, g + w, d]")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "one dtype for q and the caches")
    _need(pos.dtype == torch.int64 and pos.shape == (B,), "pos must be int64 [batch]")
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if lse is not None:
        _dev_tensor(lse, "lse")
        _need(lse.shape == (B, H) and lse.dtype == torch.float32, "lse must be fp32 [batch, heads]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rc = lib().swa_decode_fwd_gqa_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), pos.data_ptr(),
                                          out.data_ptr(), lse.data_ptr() if lse is not None else None, B, H, Hkv, d,
                                          int(w), int(g), float(scale), float(sink_bias), _dtype_code(q), _stream(q))
    if rc != 0:
        raise SwaError(rc, "swa_decode_fwd_gqa_noalloc")
    return out


def decode_scratch_bytes() -> int:
    return int(lib().swa_decode_scratch_bytes())


def _prefill_shapes(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name)
    _need(q.dim() == 4 and k.dim() == 4 and k.shape == v.shape, "q, k, v must be 4-d, k and v one shape")
    _need(q.shape[0] == k.shape[0] and q.shape[2:] == k.shape[2:],
          "q [batch, heads, n, d] and k, v [batch, kv_heads, n, d] must agree on batch, n, d")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share one dtype")
    B, H, n, d = q.shape
    return B, H, k.shape[1], n, d


def dilated_prefill(q, k, v, w: int, r: int, scale: float | None = None, return_lse: bool = False, out=None):
    """Dilated causal window: query i reads keys i, i-r, ..., i-(w-1)r."""
    import torch

    B, H, Hkv, n, d = _prefill_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    _dev_tensor(o, "out")
    _need(o.shape == q.shape and o.dtype == q.dtype, "out must match q")
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device) if return_lse else None
    rc = lib().swa_dilated_prefill_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr() if lse is not None else None, B, H, Hkv, n, d, int(w), int(r),
                                       float(scale), _dtype_code(q), _stream(q))
    if rc != 0:
        raise SwaError(rc, "swa_dilated_prefill_fwd")
    return (o, lse) if return_lse else o


def landmark_workspace_bytes(batch: int, heads: int, n: int, d: int, dtype_code: int) -> int:
    return int(lib().swa_landmark_workspace_bytes(batch, heads, n, d, dtype_code))


def landmark_prefill(q, k, v, w: int, r: int, g: int = 0, scale: float | None = None, sink_bias: float = 0.0,
                     return_lse: bool = False, out=None, workspace=None):
    """Window of w, sinks 0..g-1 and landmarks every r positions, each key once."""
    import torch

    B, H, Hkv, n, d = _prefill_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    _dev_tensor(o, "out")
    _need(o.shape == q.shape and o.dtype == q.dtype, "out must match q")
    lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device) if return_lse else None
    need = landmark_workspace_bytes(B, H, n, d, _dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    rc = lib().swa_landmark_prefill_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        lse.data_ptr() if lse is not None else None, B, H, Hkv, n, d, int(w), int(g),
                                        int(r), float(scale), float(sink_bias), _dtype_code(q), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream(q))
    if rc != 0:
        raise SwaError(rc, "swa_landmark_prefill_fwd")
    return (o, lse) if return_lse else o


KEYS = {"all": 0, "cache": 1, "chunk": 2}


def chunk_prefill(q, k_new, v_new, k_cache, v_cache, pos, w: int, g: int = 0, scale: float | None = None,
                  sink_bias: float = 0.0, keys: str = "all", return_lse: bool = False, out=None):
    """Chunked prefill against the rolling cache: q [batch, heads, t, d] at
    positions pos[b] .. pos[b]+t-1, the chunk's own k_new, v_new [batch,
    kv_heads, t, d] and caches [batch, kv_heads, g + w, d] holding positions
    < pos[b].  keys: "all", or the partial over "cache" or "chunk" keys."""
    import torch

    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("pos", pos)):
        _dev_tensor(t, name)
    _need(q.dim() == 4 and k_new.dim() == 4 and k_new.shape == v_new.shape, "q, k_new, v_new must be 4-d")
    B, H, t, d = q.shape
    Hkv = k_new.shape[1]
    _need(k_new.shape == (B, Hkv, t, d), "k_new, v_new must be [batch, kv_heads, t, d]")
    _need(k_cache.shape == v_cache.shape == (B, Hkv, g + w, d), "caches must be [batch, kv_heads, g + w, d]")
    _need(q.dtype == k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype, "one dtype for every tensor")
    _need(pos.dtype == torch.int64 and pos.shape == (B,), "pos must be int64 [batch]")
    _need(keys in KEYS, "keys must be 'all', 'cache' or 'chunk'")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    _dev_tensor(o, "out")
    _need(o.shape == q.shape and o.dtype == q.dtype, "out must match q")
    lse = torch.empty((B, H, t), dtype=torch.float32, device=q.device) if return_lse else None
    rc = lib().swa_chunk_prefill_fwd(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                                     v_cache.data_ptr(), pos.data_ptr(), o.data_ptr(),
                                     lse.data_ptr() if lse is not None else None, B, H, Hkv, t, d, int(w), int(g),
                                     float(scale), float(sink_bias), KEYS[keys], _dtype_code(q), _stream(q))
    if rc != 0:
        raise SwaError(rc, "swa_chunk_prefill_fwd")
    return (o, lse) if return_lse else o


def lse_merge(o_a, lse_a, o_b, lse_b, return_lse: bool = True, out=None):
    """Merge two partial attentions of the same rows over disjoint key sets:
    o_* [..., d] with lse_* [...] fp32."""
    import torch

    for name, t in (("o_a", o_a), ("lse_a", lse_a), ("o_b", o_b), ("lse_b", lse_b)):
        _dev_tensor(t, name)
    _need(o_a.shape == o_b.shape and o_a.dtype == o_b.dtype, "o_a and o_b must match")
    _need(lse_a.shape == lse_b.shape == o_a.shape[:-1], "lse_a, lse_b must be o's shape without d")
    _need(lse_a.dtype == lse_b.dtype == torch.float32, "lse must be fp32")
    d = o_a.shape[-1]
    rows = o_a.numel() // d
    o = torch.empty_like(o_a) if out is None else out
    _dev_tensor(o, "out")
    _need(o.shape == o_a.shape and o.dtype == o_a.dtype, "out must match o_a")
    lse = torch.empty_like(lse_a) if return_lse else None
    rc = lib().swa_lse_merge(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(), o.data_ptr(),
                             lse.data_ptr() if lse is not None else None, rows, d, _dtype_code(o_a), _stream(o_a))
    if rc != 0:
        raise SwaError(rc, "swa_lse_merge")
    return (o, lse) if return_lse else o


def band_tiles(n: int, w: int, g: int, bq: int, bk: int) -> np.ndarray:
    """The prefill tile schedule as an int array [tiles, 3] = (query block, key block, is_full)."""
    L = lib()
    count = L.swa_band_tiles(n, w, g, bq, bk, None, 0)
    if count < 0:
        raise SwaError(count, "swa_band_tiles")
    out = np.zeros((max(count, 1), 3), dtype=np.int32)
    got = L.swa_band_tiles(n, w, g, bq, bk, out.ctypes.data, count)
    if got != count:
        raise SwaError(got, "swa_band_tiles")
    return out[:count]


def prefill_tile_shape(dtype_code: int, d: int):
    bq, bk = _int(), _int()
    rc = lib().swa_prefill_tile_shape(dtype_code, d, ctypes.byref(bq), ctypes.byref(bk))
    if rc != 0:
        raise SwaError(rc, "swa_prefill_tile_shape")
    return bq.value, bk.value


def prefill_order(units: int, nqb: int, group: int = 1) -> np.ndarray:
    """Workgroup id -> (unit, query block) of a prefill launch, as int array
    [units*nqb, 2]; group = query heads per key/value head."""
    total = units * nqb
    out = np.zeros((total, 2), dtype=np.int32)
    got = lib().swa_prefill_order(units, nqb, group, out.ctypes.data, total)
    if got != total:
        raise SwaError(got, "swa_prefill_order")
    return out


def probe_mfma_bf16(out, workgroups: int, iters: int) -> float:
    """Enqueue the dense bf16 MFMA stream (measurement kernel) on out's
    device; out: float32 [workgroups * 256].  Returns its FLOP count."""
    _dev_tensor(out, "out")
    _need(out.dtype.is_floating_point and out.element_size() == 4 and out.numel() >= workgroups * 256,
          "out must be float32 with workgroups * 256 elements")
    rc = lib().swa_probe_mfma_bf16(out.data_ptr(), int(workgroups), int(iters), _stream(out))
    if rc != 0:
        raise SwaError(rc, "swa_probe_mfma_bf16")
    return float(lib().swa_probe_mfma_bf16_flops(int(workgroups), int(iters)))


def probe_hbm_read(buf, workgroups: int, streams: int, sink) -> int:
    """Enqueue the streaming read of buf (measurement kernel); sink: int32
    [workgroups].  Returns the bytes read."""
    _dev_tensor(buf, "buf")
    _dev_tensor(sink, "sink")
    _need(sink.element_size() == 4 and sink.numel() >= workgroups, "sink must hold workgroups 32-bit words")
    nbytes = buf.numel() * buf.element_size()
    rc = lib().swa_probe_hbm_read(buf.data_ptr(), nbytes, int(workgroups), int(streams), sink.data_ptr(),
                                  _stream(buf))
    if rc != 0:
        raise SwaError(rc, "swa_probe_hbm_read")
    return nbytes
