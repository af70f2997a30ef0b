"""libswa.so loads, exports every entry point that include/*.h declares, and rejects
invalid arguments before launching anything.  CPU only: every call here
fails validation, so no device work is enqueued."""
import ctypes
import os
import re

import pytest

import block_sparse_causal_band_amd as swa
from block_sparse_causal_band_amd import binding

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))

OK, EINVAL, EUNSUP, EALIGN, EHIP, EWS, ESCRATCH = 0, -1, -2, -3, -4, -5, -6
P = 4096  # a fake, 16-byte aligned "device pointer": never dereferenced on these paths


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(swa_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("swa_prefill_fwd", "swa_decode_fwd", "swa_kv_append", "swa_decode_workspace_bytes",
                 "swa_strerror", "swa_band_tiles"):
        assert want in names


def test_headers_declare_the_measurement_probes():
    assert {"swa_probe_mfma_bf16", "swa_probe_mfma_bf16_flops", "swa_probe_hbm_read"} <= set(declared_functions())


def test_probe_rejects_and_counts():
    L = swa.lib()
    assert L.swa_probe_mfma_bf16(None, 1, 1, None) == EINVAL
    assert L.swa_probe_mfma_bf16(P, 0, 1, None) == EINVAL
    assert L.swa_probe_mfma_bf16(P + 2, 1, 1, None) == EALIGN
    assert L.swa_probe_mfma_bf16_flops(3, 5) == 3 * 4 * 5 * 4 * 32768
    assert L.swa_probe_mfma_bf16_flops(0, 5) == 0
    assert L.swa_probe_hbm_read(P, 32768 * 4, 4, 3, P, None) == EINVAL       # streams
    assert L.swa_probe_hbm_read(P, 32768 * 4 + 16, 4, 2, P, None) == EINVAL  # not whole rounds
    assert L.swa_probe_hbm_read(P + 8, 32768 * 4, 4, 2, P, None) == EALIGN


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), f"{name} not exported"


def test_strerror_covers_every_status():
    for st in (OK, EINVAL, EUNSUP, EALIGN, EHIP, EWS, ESCRATCH):
        assert swa.strerror(st) and swa.strerror(st) != "unknown status"
    assert swa.strerror(-99) == "unknown status"


def _prefill(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, batch=1, heads=1, n=16, d=128, w=4, g=0,
             scale=0.125, bias=0.0, dtype=1)
    a.update(kw)
    return swa.lib().swa_prefill_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["batch"], a["heads"], a["n"],
                                     a["d"], a["w"], a["g"], a["scale"], a["bias"], a["dtype"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), EINVAL), (dict(k=None), EINVAL), (dict(v=None), EINVAL), (dict(o=None), EINVAL),
    (dict(batch=0), EINVAL), (dict(heads=0), EINVAL), (dict(n=0), EINVAL), (dict(w=0), EINVAL),
    (dict(g=-1), EINVAL), (dict(scale=0.0), EINVAL), (dict(scale=-1.0), EINVAL),
    (dict(scale=float("nan")), EINVAL), (dict(scale=float("inf")), EINVAL), (dict(bias=float("nan")), EINVAL),
    (dict(d=96), EUNSUP), (dict(d=256), EUNSUP), (dict(dtype=7), EUNSUP),
    (dict(q=P + 8), EALIGN), (dict(o=P + 2), EALIGN), (dict(lse=P + 2), EALIGN),
    (dict(n=2**31 - 100), EINVAL),
])
def test_prefill_rejects(kw, want):
    assert _prefill(**kw) == want


def _append(**kw):
    a = dict(kc=P, vc=P, kn=P, vn=P, pos=P, batch=1, heads=1, t=1, d=128, w=8, g=0, dtype=1)
    a.update(kw)
    return swa.lib().swa_kv_append(a["kc"], a["vc"], a["kn"], a["vn"], a["pos"], a["batch"], a["heads"], a["t"],
                                   a["d"], a["w"], a["g"], a["dtype"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(kc=None), EINVAL), (dict(pos=None), EINVAL), (dict(batch=0), EINVAL), (dict(t=-1), EINVAL),
    (dict(w=0), EINVAL), (dict(g=-2), EINVAL), (dict(d=32), EUNSUP), (dict(dtype=3), EUNSUP),
    (dict(kn=P + 4), EALIGN), (dict(pos=P + 4), EALIGN),
    (dict(t=0), OK),  # nothing to write: returns without launching
])
def test_kv_append_rejects(kw, want):
    assert _append(**kw) == want


def _decode(**kw):
    a = dict(q=P, kc=P, vc=P, pos=P, o=P, lse=None, batch=64, heads=32, d=128, w=4096, g=4,
             scale=0.125, bias=0.0, dtype=1, ws=None, wsb=0)
    a.update(kw)
    return swa.lib().swa_decode_fwd(a["q"], a["kc"], a["vc"], a["pos"], a["o"], a["lse"], a["batch"], a["heads"],
                                    a["d"], a["w"], a["g"], a["scale"], a["bias"], a["dtype"], a["ws"], a["wsb"],
                                    None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), EINVAL), (dict(kc=None), EINVAL), (dict(pos=None), EINVAL), (dict(o=None), EINVAL),
    (dict(batch=0), EINVAL), (dict(w=0), EINVAL), (dict(g=-1), EINVAL), (dict(scale=0.0), EINVAL),
    (dict(d=80), EUNSUP), (dict(dtype=2), EUNSUP), (dict(vc=P + 8), EALIGN), (dict(lse=P + 1), EALIGN),
    (dict(batch=1, heads=1), EWS),            # small problem splits the cache -> needs a workspace
    (dict(batch=1, heads=1, ws=P, wsb=8), EWS),
])
def test_decode_rejects(kw, want):
    assert _decode(**kw) == want


def test_decode_workspace_sizes():
    assert swa.decode_workspace_bytes(64, 32, 128, 4096, 4) == 0      # enough (batch, head) pairs
    need = swa.decode_workspace_bytes(1, 1, 128, 4096, 4)
    assert need > 0 and need % 16 == 0
    assert swa.decode_workspace_bytes(1, 1, 96, 4096, 4) == 0           # unsupported d: nothing to size


def _decode_noalloc(**kw):
    a = dict(q=P, kc=P, vc=P, pos=P, o=P, lse=None, batch=64, heads=32, kv_heads=8, d=128, w=4096, g=4,
             scale=0.125, bias=0.0, dtype=1)
    a.update(kw)
    return swa.lib().swa_decode_fwd_gqa_noalloc(a["q"], a["kc"], a["vc"], a["pos"], a["o"], a["lse"], a["batch"],
                                                a["heads"], a["kv_heads"], a["d"], a["w"], a["g"], a["scale"],
                                                a["bias"], a["dtype"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), EINVAL), (dict(kc=None), EINVAL), (dict(vc=None), EINVAL), (dict(pos=None), EINVAL),
    (dict(o=None), EINVAL), (dict(batch=0), EINVAL), (dict(heads=0), EINVAL), (dict(kv_heads=3), EINVAL),
    (dict(w=0), EINVAL), (dict(g=-1), EINVAL), (dict(scale=0.0), EINVAL), (dict(bias=float("inf")), EINVAL),
    (dict(w=2**31 - 8), EINVAL), (dict(d=80), EUNSUP), (dict(dtype=2), EUNSUP),
    (dict(q=P + 8), EALIGN), (dict(pos=P + 4), EALIGN), (dict(lse=P + 2), EALIGN),
])
def test_decode_noalloc_rejects(kw, want):
    assert _decode_noalloc(**kw) == want


def test_decode_scratch_covers_every_split():
    """The fixed scratch of the allocation-free decode holds the partial
    records of every shape the split rule can produce: the records peak just
    below the job counts at which a launch stops splitting, so sweep those
    (and a coarse grid) over every group size, both head dims and short and
    long caches; the workspace size here is the largest any kernel needs."""
    L = swa.lib()
    cap = int(L.swa_decode_scratch_bytes())
    assert cap == 16 << 20
    worst = 0
    for d in (64, 128):
        for group in (1, 2, 3, 4, 8, 16, 32):
            for kvh in list(range(1, 80)) + [127, 128, 255, 256, 511, 512, 1023, 1024, 2047]:
                heads = kvh * group
                for rows in (256, 1028, 4100, 65540):
                    need = int(L.swa_decode_workspace_bytes_gqa(1, heads, kvh, d, rows - 4, 4))
                    worst = max(worst, need)
                    assert need <= cap, (d, group, heads, rows, need)
    assert worst > (1 << 20)  # the sweep reaches the large splits


def _prefill_gqa(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, batch=1, heads=8, kv_heads=2, n=16, d=128, w=4, g=0,
             scale=0.125, bias=0.0, dtype=1)
    a.update(kw)
    return swa.lib().swa_prefill_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["batch"], a["heads"],
                                         a["kv_heads"], a["n"], a["d"], a["w"], a["g"], a["scale"], a["bias"],
                                         a["dtype"], None)


def _decode_gqa(**kw):
    a = dict(q=P, kc=P, vc=P, pos=P, o=P, lse=None, batch=64, heads=32, kv_heads=8, d=128, w=4096, g=4,
             scale=0.125, bias=0.0, dtype=1, ws=None, wsb=0)
    a.update(kw)
    return swa.lib().swa_decode_fwd_gqa(a["q"], a["kc"], a["vc"], a["pos"], a["o"], a["lse"], a["batch"],
                                        a["heads"], a["kv_heads"], a["d"], a["w"], a["g"], a["scale"], a["bias"],
                                        a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(kv_heads=0), EINVAL), (dict(kv_heads=3), EINVAL), (dict(kv_heads=16), EINVAL),
    (dict(kv_heads=-2), EINVAL), (dict(k=None), EINVAL), (dict(d=80), EUNSUP), (dict(v=P + 8), EALIGN),
])
def test_prefill_gqa_rejects(kw, want):
    assert _prefill_gqa(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(kv_heads=0), EINVAL), (dict(kv_heads=5), EINVAL), (dict(kv_heads=64), EINVAL),
    (dict(kc=None), EINVAL), (dict(dtype=2), EUNSUP),
    (dict(batch=1, heads=8, kv_heads=1), EWS),  # one workgroup's worth of heads: split, needs a workspace
])
def test_decode_gqa_rejects(kw, want):
    assert _decode_gqa(**kw) == want


def test_decode_gqa_workspace_sizes():
    # 64 x 32 query heads in groups of 4: 512 workgroups of 4 heads -> split in 4 (at least 256 rows each)
    assert swa.decode_workspace_bytes(64, 32, 128, 4096, 4, kv_heads=8) == 64 * 32 * 4 * (2 + 128) * 4
    assert swa.decode_workspace_bytes(64, 32, 128, 4096, 4, kv_heads=32) == 0
    assert swa.decode_workspace_bytes(64, 32, 128, 4096, 4, kv_heads=5) == 0   # invalid grouping
    # one key/value head for 8 query heads at batch 1: one job, 16 splits
    assert swa.decode_workspace_bytes(1, 8, 128, 4096, 4, kv_heads=1) == 8 * 16 * (2 + 128) * 4


def _chunk(**kw):
    a = dict(q=P, kn=P, vn=P, kc=P, vc=P, pos=P, o=P, lse=None, batch=1, heads=2, kv_heads=2, t=16, d=128, w=8,
             g=0, scale=0.125, bias=0.0, keys=0, dtype=1)
    a.update(kw)
    return swa.lib().swa_chunk_prefill_fwd(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["pos"], a["o"], a["lse"],
                                           a["batch"], a["heads"], a["kv_heads"], a["t"], a["d"], a["w"], a["g"],
                                           a["scale"], a["bias"], a["keys"], a["dtype"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), EINVAL), (dict(kc=None), EINVAL), (dict(pos=None), EINVAL), (dict(o=None), EINVAL),
    (dict(t=0), EINVAL), (dict(batch=0), EINVAL), (dict(w=0), EINVAL), (dict(g=-1), EINVAL),
    (dict(keys=3), EINVAL), (dict(keys=-1), EINVAL), (dict(kv_heads=3), EINVAL), (dict(kv_heads=0), EINVAL),
    (dict(scale=0.0), EINVAL), (dict(bias=float("inf")), EINVAL), (dict(t=1 << 24), EINVAL),
    (dict(d=80), EUNSUP), (dict(dtype=5), EUNSUP),
    (dict(kc=P + 8), EALIGN), (dict(vn=P + 4), EALIGN), (dict(pos=P + 4), EALIGN), (dict(lse=P + 2), EALIGN),
])
def test_chunk_prefill_rejects(kw, want):
    assert _chunk(**kw) == want


def _merge(**kw):
    a = dict(oa=P, la=P, ob=P, lb=P, o=P, lse=None, rows=4, d=128, dtype=1)
    a.update(kw)
    return swa.lib().swa_lse_merge(a["oa"], a["la"], a["ob"], a["lb"], a["o"], a["lse"], a["rows"], a["d"],
                                   a["dtype"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(oa=None), EINVAL), (dict(lb=None), EINVAL), (dict(o=None), EINVAL), (dict(rows=0), EINVAL),
    (dict(d=96), EUNSUP), (dict(dtype=9), EUNSUP), (dict(la=P + 2), EALIGN), (dict(ob=P + 8), EALIGN),
])
def test_lse_merge_rejects(kw, want):
    assert _merge(**kw) == want


def _append_fp8(**kw):
    a = dict(kc=P, vc=P, kn=P, vn=P, pos=P, ks=P, vs=P, batch=1, heads=1, t=1, d=128, w=8, g=0, dtype=1)
    a.update(kw)
    return swa.lib().swa_kv_append_fp8(a["kc"], a["vc"], a["kn"], a["vn"], a["pos"], a["ks"], a["vs"], a["batch"],
                                       a["heads"], a["t"], a["d"], a["w"], a["g"], a["dtype"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(kc=None), EINVAL), (dict(ks=None), EINVAL), (dict(vs=None), EINVAL), (dict(batch=0), EINVAL),
    (dict(t=-1), EINVAL), (dict(w=0), EINVAL), (dict(d=32), EUNSUP), (dict(dtype=3), EUNSUP),
    (dict(ks=P + 2), EALIGN), (dict(pos=P + 4), EALIGN), (dict(kn=P + 8), EALIGN),
    (dict(t=0), OK),
])
def test_kv_append_fp8_rejects(kw, want):
    assert _append_fp8(**kw) == want


def _decode_fp8(**kw):
    a = dict(q=P, kc=P, vc=P, ks=P, vs=P, pos=P, o=P, lse=None, batch=64, heads=32, kv_heads=32, d=128, w=4096,
             g=4, scale=0.125, bias=0.0, dtype=1, ws=None, wsb=0)
    a.update(kw)
    return swa.lib().swa_decode_fwd_fp8(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["pos"], a["o"], a["lse"],
                                        a["batch"], a["heads"], a["kv_heads"], a["d"], a["w"], a["g"], a["scale"],
                                        a["bias"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), EINVAL), (dict(ks=None), EINVAL), (dict(vs=None), EINVAL), (dict(kv_heads=3), EINVAL),
    (dict(w=0), EINVAL), (dict(scale=-1.0), EINVAL), (dict(d=96), EUNSUP), (dict(dtype=2), EUNSUP),
    (dict(vs=P + 1), EALIGN), (dict(kc=P + 8), EALIGN),
    (dict(batch=1, heads=8, kv_heads=1), EWS),
])
def test_decode_fp8_rejects(kw, want):
    assert _decode_fp8(**kw) == want



def _dilated(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, batch=1, heads=2, kv_heads=2, n=64, d=128, w=4, r=2, scale=0.125,
             dtype=1)
    a.update(kw)
    return swa.lib().swa_dilated_prefill_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["batch"], a["heads"],
                                             a["kv_heads"], a["n"], a["d"], a["w"], a["r"], a["scale"], a["dtype"],
                                             None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), EINVAL), (dict(r=0), EINVAL), (dict(w=0), EINVAL), (dict(n=0), EINVAL),
    (dict(kv_heads=3), EINVAL), (dict(d=48), EUNSUP), (dict(o=P + 4), EALIGN),
])
def test_dilated_rejects(kw, want):
    assert _dilated(**kw) == want


def _landmark(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, batch=1, heads=2, kv_heads=2, n=64, d=128, w=4, g=0, r=2, scale=0.125,
             bias=0.0, dtype=1, ws=P, wsb=1 << 30)
    a.update(kw)
    return swa.lib().swa_landmark_prefill_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["batch"], a["heads"],
                                              a["kv_heads"], a["n"], a["d"], a["w"], a["g"], a["r"], a["scale"],
                                              a["bias"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), EINVAL), (dict(r=0), EINVAL), (dict(g=-1), EINVAL), (dict(bias=float("nan")), EINVAL),
    (dict(d=48), EUNSUP),
    # fp32 merges through the workspace (bf16 needs none)
    (dict(ws=None, dtype=0), EWS), (dict(wsb=100, dtype=0), EWS), (dict(ws=P + 8, dtype=0), EALIGN),
])
def test_landmark_rejects(kw, want):
    assert _landmark(**kw) == want


def test_landmark_workspace_size():
    # bf16: none (one launch over landmark, window and sink tiles); fp32: the
    # landmark part's o plus two lse rows, each rounded up to 256 bytes
    assert swa.landmark_workspace_bytes(1, 2, 64, 128, 1) == 0
    assert swa.landmark_workspace_bytes(1, 2, 64, 128, 0) == 1 * 2 * 64 * 128 * 4 + 2 * 512
    assert swa.landmark_workspace_bytes(1, 2, 64, 96, 1) == 0


def test_row_byte_limits():
    # one (batch, head)'s rows are addressed with 32-bit byte offsets
    assert _prefill(n=(1 << 24), d=128, dtype=1) == EINVAL            # 2^24 rows x 256 B = 2^32
    assert _prefill(n=(1 << 23), d=128, dtype=0) == EINVAL            # fp32: 2^23 x 512 B
    assert _decode(w=(1 << 23), g=0, d=128) == EINVAL                  # cache rows x d x 4 >= 2^32
    assert _decode_fp8(w=(1 << 23), g=0, d=128) == EINVAL
