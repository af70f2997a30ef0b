"""The rolling-buffer cache model and the decode oracle (CPU only)."""
import numpy as np
import pytest

from oracle import cache_model
from tests import oracle_pins as pins


def _append_positions(last, w, g, d=1):
    """Append positions 0..last one at a time; value of position t is t."""
    kc = np.full((1, 1, g + w, d), -1.0)
    vc = np.full((1, 1, g + w, d), -1.0)
    for t in range(last + 1):
        val = np.full((1, 1, 1, d), float(t))
        cache_model.append(kc, vc, val, val, [t], w, g)
    return kc, vc


@pytest.mark.parametrize("w,g,last,slots", pins.golden_fig4())
def test_fig4_ring_state(w, g, last, slots):
    kc, vc = _append_positions(last, w, g)
    ring = kc[0, 0, g:, 0].astype(int).tolist()
    assert ring == slots
    assert vc[0, 0, g:, 0].astype(int).tolist() == slots


def test_fig4_eviction_of_p5():
    """Moving from p7 to p8 with w=3 discards p5 and keeps the latest three."""
    kc7, _ = _append_positions(7, 3, 0)
    kc8, _ = _append_positions(8, 3, 0)
    assert 5 in kc7[0, 0, :, 0].astype(int).tolist()
    assert 5 not in kc8[0, 0, :, 0].astype(int).tolist()
    assert sorted(kc8[0, 0, :, 0].astype(int).tolist()) == [6, 7, 8]


def test_sinks_stay_after_leaving_the_window():
    """A position that is always read must remain stored (Figure 4 text)."""
    w, g = 3, 2
    kc, _ = _append_positions(20, w, g)
    assert kc[0, 0, :g, 0].astype(int).tolist() == [0, 1]
    assert sorted(kc[0, 0, g:, 0].astype(int).tolist()) == [18, 19, 20]


@pytest.mark.parametrize("T", [1, 2, 5, 7, 12, 30])
def test_multi_token_append_equals_one_by_one(T):
    w, g, d = 5, 3, 2
    rng = np.random.default_rng(T)
    for start in (0, 1, 4, 9, 23):
        new_k = rng.standard_normal((2, 2, T, d))
        new_v = rng.standard_normal((2, 2, T, d))
        a_k = np.zeros((2, 2, g + w, d)); a_v = np.zeros_like(a_k)
        b_k = np.zeros_like(a_k); b_v = np.zeros_like(a_k)
        cache_model.append(a_k, a_v, new_k, new_v, [start, start + 2], w, g)
        for t in range(T):
            cache_model.append(b_k, b_v, new_k[:, :, t:t + 1], new_v[:, :, t:t + 1],
                               [start + t, start + 2 + t], w, g)
        assert np.array_equal(a_k, b_k) and np.array_equal(a_v, b_v)


@pytest.mark.parametrize("w,g", [(1, 0), (3, 1), (4, 4), (6, 2), (5, 0), (2, 7)])
def test_logical_rows_cover_attended_set_once(orc, w, g):
    for p in range(0, 3 * (w + g) + 2):
        positions, rows = cache_model.logical_rows(p, w, g)
        assert len(set(positions.tolist())) == len(positions)
        assert sorted(positions.tolist()) == [j for j in range(p + 1) if orc.attended(p, j, w, g)]
        assert np.all(rows >= 0) and np.all(rows < g + w)


@pytest.mark.parametrize("w,g,beta", [(4, 2, 0.0), (4, 2, 4.0), (1, 0, 0.0), (7, 3, -1.0), (3, 5, 2.0)])
def test_decode_through_cache_equals_prefill_row(orc, w, g, beta):
    """Append positions 0..p into the cache, read the cache back by logical
    position, and decode: equals row p of prefill over the whole sequence."""
    rng = np.random.default_rng(w * 10 + g)
    n, d, H = 3 * (w + g) + 3, 4, 2
    q, k, v = (rng.standard_normal((1, H, n, d)) for _ in range(3))
    kc = np.zeros((1, H, g + w, d)); vc = np.zeros_like(kc)
    o_ref, lse_ref = orc.prefill(q, k, v, w=w, g=g, beta=beta)
    for p in range(n):
        cache_model.append(kc, vc, k[:, :, p:p + 1], v[:, :, p:p + 1], [p], w, g)
        positions, rows = cache_model.logical_rows(p, w, g)
        kpos = np.tile(positions, (H, 1))
        ks = kc[0][:, rows]
        vs = vc[0][:, rows]
        o, lse = orc.decode(q[0, :, p], [p] * H, kpos, ks, vs, w=w, g=g, beta=beta)
        assert np.max(np.abs(o - o_ref[0, :, p])) < 1e-13
        assert np.max(np.abs(lse - lse_ref[0, :, p])) < 1e-13
