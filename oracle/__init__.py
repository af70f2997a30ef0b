"""fp64 CPU oracle for exact causal sliding-window attention with sinks.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite, the
smoke check (``__graft_entry__.smoke``) and the benchmark's ``cpu_baseline``
leg may import this package.  It shares no code with the HIP library under
``block_sparse_causal_band_amd/``; the two are independent implementations
of the same definition, so that one can check the other.

Contents
  * ``swa_oracle.c`` (loaded here through ctypes): the dense fp64 definition
    -- attended-set predicate, pair counts, connectivity grid, prefill rows,
    decode over the logical sequence.
  * ``brute.py``: a second, set-based pure-Python evaluation for tiny inputs.
  * ``cache_model.py``: the rolling-buffer cache written token by token.

Sources (page title, then the section / figure used):
  * "Sliding Window and Sparse Attention, from Longformer to CSA2":
    s1 (scaled dot-product attention, causal rule), s2 (window i-w+1..i,
    rolling buffer slot i mod w, attention sinks), s10 glossary (LSE).
  * "Local and Sparse Attention: Reading Fewer Token Positions": Figures 1, 2
    and 4 and the text between them (window of 3 counts the current token;
    -inf masking, not zeroing; anchor union read once; eviction).
  * "Sliding Window and Sparse Attention, from Longformer to CSA2", s10
    glossary, GQA: several query heads share one key/value head.  The page
    does not say which ones; the reading taken here is consecutive groups,
    query head h of H reading key/value head h // (H / Hkv) (``kv_head_of``).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "swa_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_c_long_p = ctypes.POINTER(ctypes.c_long)
_c_double_p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, IEEE semantics kept)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall", "-o", tmp, SOURCE]
        )
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Oracle:
    """ctypes view of one build of ``swa_oracle.c`` (the default one, or a
    copy compiled elsewhere, e.g. by a test that plants a mistake in it)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        L.swa_oracle_attended.argtypes = [ctypes.c_long] * 4
        L.swa_oracle_attended.restype = ctypes.c_int
        L.swa_oracle_row_count.argtypes = [ctypes.c_long] * 3
        L.swa_oracle_row_count.restype = ctypes.c_long
        L.swa_oracle_pair_count.argtypes = [ctypes.c_long] * 3
        L.swa_oracle_pair_count.restype = ctypes.c_long
        L.swa_oracle_mask.argtypes = [ctypes.c_long] * 3 + [ctypes.c_void_p]
        L.swa_oracle_mask.restype = ctypes.c_int
        L.swa_oracle_prefill.argtypes = [
            _c_double_p, _c_double_p, _c_double_p,
            ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            ctypes.c_double, ctypes.c_double, _c_long_p, ctypes.c_long,
            _c_double_p, _c_double_p, ctypes.c_int,
        ]
        L.swa_oracle_prefill.restype = ctypes.c_int
        L.swa_oracle_decode.argtypes = [
            _c_double_p, _c_long_p, _c_long_p, _c_double_p, _c_double_p,
            ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            ctypes.c_double, ctypes.c_double, _c_double_p, _c_double_p, ctypes.c_int,
        ]
        L.swa_oracle_decode.restype = ctypes.c_int
        L.swa_oracle_num_threads.argtypes = []
        L.swa_oracle_num_threads.restype = ctypes.c_int
        self.L = L
        self.path = path

    def attended(self, i: int, j: int, w: int, g: int) -> bool:
        return bool(self.L.swa_oracle_attended(i, j, w, g))

    def row_count(self, i: int, w: int, g: int) -> int:
        return int(self.L.swa_oracle_row_count(i, w, g))

    def pair_count(self, n: int, w: int, g: int) -> int:
        return int(self.L.swa_oracle_pair_count(n, w, g))

    def mask(self, n: int, w: int, g: int) -> np.ndarray:
        out = np.zeros((n, n), dtype=np.uint8)
        if self.L.swa_oracle_mask(n, w, g, out.ctypes.data) != 0:
            raise ValueError("swa_oracle_mask failed")
        return out

    def num_threads(self) -> int:
        return int(self.L.swa_oracle_num_threads())

    def prefill(self, q, k, v, w: int, g: int = 0, scale: float | None = None,
                beta: float = 0.0, rows=None, nthreads: int = 0):
        """Rows of causal sliding-window attention with sinks, in fp64.

        q, k, v: [..., n, d] (any leading batch/head dims).  ``rows``: the query
        rows to evaluate (default: all).  Returns (o [..., nrows, d], lse [..., nrows]).
        Grouped-query attention: q [..., H, n, d] with k, v [..., Hkv, n, d],
        Hkv dividing H; each query head is paired with its key/value head
        (``kv_head_of``) before the rows are evaluated.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        if k.shape == v.shape and k.shape != q.shape and q.ndim >= 3:
            k, v = expand_kv_heads(q.shape[-3], k), expand_kv_heads(q.shape[-3], v)
        if q.shape != k.shape or q.shape != v.shape or q.ndim < 2:
            raise ValueError("q, k, v must share one shape [..., n, d]")
        lead = q.shape[:-2]
        n, d = q.shape[-2:]
        bh = int(np.prod(lead)) if lead else 1
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        r = np.arange(n) if rows is None else np.asarray(rows)
        r = np.ascontiguousarray(r.astype(np.int_))
        nrows = r.shape[0]
        o = np.zeros((bh, nrows, d), dtype=np.float64)
        lse = np.zeros((bh, nrows), dtype=np.float64)
        rc = self.L.swa_oracle_prefill(
            _dp(q), _dp(k), _dp(v), bh, n, d, w, g, float(scale), float(beta),
            _lp(r), nrows, _dp(o), _dp(lse), int(nthreads),
        )
        if rc != 0:
            raise ValueError(f"swa_oracle_prefill failed ({rc})")
        return o.reshape(*lead, nrows, d), lse.reshape(*lead, nrows)

    def decode(self, q, p, kpos, k, v, w: int, g: int = 0, scale: float | None = None,
               beta: float = 0.0, nthreads: int = 0):
        """One query per unit at logical position p, over supplied logical rows.

        q: [U, d]; p: [U]; kpos: [U, nk] logical positions (<0 = padding);
        k, v: [U, nk, d].  Raises if a unit's rows do not cover its attended set
        exactly once.  Returns (o [U, d], lse [U]).
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        p = np.ascontiguousarray(np.asarray(p).astype(np.int_))
        kpos = np.ascontiguousarray(np.asarray(kpos).astype(np.int_))
        U, d = q.shape
        nk = kpos.shape[1]
        if k.shape != (U, nk, d) or v.shape != (U, nk, d) or p.shape != (U,):
            raise ValueError("shape mismatch")
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        o = np.zeros((U, d), dtype=np.float64)
        lse = np.zeros((U,), dtype=np.float64)
        rc = self.L.swa_oracle_decode(
            _dp(q), _lp(p), _lp(kpos), _dp(k), _dp(v), U, nk, d, w, g,
            float(scale), float(beta), _dp(o), _dp(lse), int(nthreads),
        )
        if rc != 0:
            raise ValueError(f"swa_oracle_decode failed ({rc})")
        return o, lse


def kv_head_of(h: int, heads: int, kv_heads: int) -> int:
    """Key/value head read by query head h when kv_heads of them serve heads
    query heads (grouped-query attention, consecutive groups)."""
    if kv_heads < 1 or heads % kv_heads != 0 or not 0 <= h < heads:
        raise ValueError("kv_heads must divide heads and 0 <= h < heads")
    return h // (heads // kv_heads)


def expand_kv_heads(heads: int, x: np.ndarray) -> np.ndarray:
    """x [..., Hkv, n, d] -> [..., heads, n, d] with query head h holding
    x[..., kv_head_of(h), :, :]."""
    kv_heads = x.shape[-3]
    idx = [kv_head_of(h, heads, kv_heads) for h in range(heads)]
    return np.ascontiguousarray(np.take(x, idx, axis=-3))


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two partial attentions of the same rows over disjoint key sets
    ("Sliding Window and Sparse Attention, from Longformer to CSA2", s10
    glossary, LSE): each part's output weighs e^lse of that part.  A part
    with lse = -inf weighs 0; two such parts give o = 0, lse = -inf.
    o_*: [..., d], lse_*: [...]; fp64 results."""
    o_a, o_b = _f64(o_a), _f64(o_b)
    lse_a, lse_b = _f64(lse_a), _f64(lse_b)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - m_safe))
    wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - m_safe))
    tot = wa + wb
    inv = np.where(tot > 0, 1.0 / np.where(tot > 0, tot, 1.0), 0.0)
    o = (wa * inv)[..., None] * o_a + (wb * inv)[..., None] * o_b
    lse = np.where(tot > 0, m_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    return o, lse


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``swa_oracle.c`` next to this file (built if absent)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        _DEFAULT = Oracle(LIB_PATH)
    return _DEFAULT


def _f64(x) -> np.ndarray:
    """Exact conversion to a contiguous fp64 array (bf16 and fp32 embed exactly)."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _dp(a: np.ndarray):
    return a.ctypes.data_as(_c_double_p)


def _lp(a: np.ndarray):
    return a.ctypes.data_as(_c_long_p)


def attended(i, j, w, g):
    return default().attended(i, j, w, g)


def row_count(i, w, g):
    return default().row_count(i, w, g)


def pair_count(n, w, g):
    return default().pair_count(n, w, g)


def mask(n, w, g):
    return default().mask(n, w, g)


def num_threads():
    return default().num_threads()


def prefill(*args, **kwargs):
    return default().prefill(*args, **kwargs)


def decode(*args, **kwargs):
    return default().decode(*args, **kwargs)
