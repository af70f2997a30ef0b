"""The prefill tile scheduler (host code of libswa.so) against the oracle's
attended-set predicate.  CPU only: the hooks launch nothing."""
import numpy as np
import pytest

import block_sparse_causal_band_amd as swa

SHAPES = [
    # (n, w, g) at awkward and at real sizes
    (8, 3, 0), (8, 3, 1), (257, 1, 0), (257, 63, 0), (257, 64, 4), (257, 65, 0), (300, 300, 0),
    (300, 1000, 2), (1000, 127, 65), (1000, 129, 130), (777, 300, 4), (64, 64, 64), (129, 5, 200),
]
TILES = [(128, 64), (64, 64), (32, 32), (128, 128), (16, 48), (256, 32)]


def _check(orc, n, w, g, bq, bk):
    tiles = swa.band_tiles(n, w, g, bq, bk)
    mask = orc.mask(n, w, g).astype(bool)
    sink = np.zeros((n, n), dtype=bool)
    sink[:, :g] = True
    seen = set()
    covered = np.zeros((n, n), dtype=bool)
    last_qb = -1
    for qb, kb, full in tiles.tolist():
        assert (qb, kb) not in seen, "tile visited twice"
        seen.add((qb, kb))
        assert qb >= last_qb, "query blocks out of order"
        last_qb = qb
        rows = slice(qb * bq, min(n, (qb + 1) * bq))
        cols = slice(kb * bk, min(n, (kb + 1) * bk))
        blk = mask[rows, cols]
        assert blk.any(), f"tile ({qb},{kb}) holds no attended pair"
        if full:
            assert (kb + 1) * bk <= n, "FULL tile past the end of the sequence"
            assert blk.all(), f"FULL tile ({qb},{kb}) has an excluded pair"
            assert not sink[rows, cols].any(), f"FULL tile ({qb},{kb}) holds a sink key"
        covered[rows, cols] = True
    assert not (mask & ~covered).any(), "an attended pair lies in no visited tile"
    # visiting order inside a query block: sink blocks first, then the band ascending
    for qb in np.unique(tiles[:, 0]):
        kbs = tiles[tiles[:, 0] == qb, 1].tolist()
        assert kbs == sorted(kbs)
    return tiles


@pytest.mark.parametrize("n,w,g", SHAPES)
@pytest.mark.parametrize("bq,bk", TILES + [(256, 64), (32, 64)])
def test_schedule_cover_minimal_full(orc, n, w, g, bq, bk):
    _check(orc, n, w, g, bq, bk)


def test_kernel_tile_shape():
    for d in (64, 128):
        assert swa.prefill_tile_shape(swa.SWA_BF16, d) == (128, 64)
        assert swa.prefill_tile_shape(swa.SWA_F32, d) == (128, 64)


def _count_closed_form(n, w, g, bq, bk):
    """Visited tiles per head from the band/sink block ranges, summed in Python."""
    total = 0
    for qb in range((n + bq - 1) // bq):
        q0, q1 = qb * bq, min(n, (qb + 1) * bq) - 1
        lo = max(0, q0 - w + 1) // bk
        hi = q1 // bk
        ns = min((g - 1) // bk + 1, lo) if g > 0 else 0
        total += ns + hi - lo + 1
    return total


@pytest.mark.parametrize("n,w,g", [(16384, 4096, 0), (32768, 4096, 4), (131072, 1024, 0)])
@pytest.mark.parametrize("bq,bk", [(128, 64), (256, 32)])
def test_real_config_tile_counts(n, w, g, bq, bk):
    tiles = swa.band_tiles(n, w, g, bq, bk)
    assert len(tiles) == _count_closed_form(n, w, g, bq, bk)
    dense_causal = sum(-(-min(n, (qb + 1) * bq) // bk) for qb in range((n + bq - 1) // bq))
    assert len(tiles) < dense_causal


@pytest.mark.parametrize("units,nqb,group", [(1, 1, 1), (1, 7, 1), (3, 5, 1), (32, 128, 1), (16, 1024, 1), (5, 13, 1),
                                              (2, 3, 1), (32, 128, 4), (32, 32, 4), (8, 5, 8), (6, 7, 3), (64, 9, 16)])
def test_workgroup_order_is_a_permutation(units, nqb, group):
    order = swa.prefill_order(units, nqb, group)
    pairs = {(u, q) for u, q in order.tolist()}
    assert len(pairs) == units * nqb
    assert pairs == {(u, q) for u in range(units) for q in range(nqb)}


def test_workgroup_order_rejects_a_group_that_does_not_divide_the_units():
    with pytest.raises(swa.SwaError):
        swa.prefill_order(6, 4, 4)


@pytest.mark.parametrize("units,nqb,group", [(32, 128, 4), (32, 32, 4), (16, 64, 2), (8, 100, 8)])
def test_grouped_query_heads_take_each_block_together(units, nqb, group):
    """With several query heads per key/value head, the group's heads take
    the same query block at consecutive logical positions on one XCD, so
    they read that block's K/V tiles from one L2 at about the same time:
    within each XCD's run the workgroups come in runs of `group`, one per
    query head of a group, all on the same block."""
    order = swa.prefill_order(units, nqb, group)
    for xcd in range(8):
        run = order[xcd::8].tolist()
        for (u0, q0), (u1, q1) in zip(run, run[1:]):
            if u1 % group != 0:  # not the first query head of its group: follows the previous head
                assert (u1, q1) == (u0 + 1, q0)
    # one key/value head's group stays on one XCD for the gqa workload shape
    if (units, nqb, group) == (32, 128, 4):
        for xcd in range(8):
            assert len({u // group for u in order[xcd::8, 0].tolist()}) == 1


def test_workgroup_order_keeps_heads_on_one_xcd():
    """Workgroups dispatched to one XCD (id % 8) get neighbouring query blocks."""
    order = swa.prefill_order(32, 128)
    for xcd in range(8):
        units = order[xcd::8, 0]
        assert len(np.unique(units)) == 4  # 32 heads x 128 blocks over 8 XCDs


def test_workgroup_order_runs_blocks_first_to_last():
    """Within each XCD's run a head's query blocks come in increasing order, so
    the low end of a block's window is what the block before it just read."""
    order = swa.prefill_order(32, 128)
    for xcd in range(8):
        run = order[xcd::8]
        for u in np.unique(run[:, 0]):
            qbs = run[run[:, 0] == u, 1]
            assert np.all(np.diff(qbs) == 1) and qbs[0] == 0


def test_schedule_random_shapes(orc):
    """The same checks over random shapes (seeded): ragged n, windows narrower
    and wider than a tile or the sequence, sinks below, inside and beyond the
    first tile."""
    rng = np.random.default_rng(2024)
    for _ in range(60):
        n = int(rng.integers(1, 400))
        w = int(rng.integers(1, 450))
        g = int(rng.integers(0, 80))
        bq, bk = TILES[int(rng.integers(0, len(TILES)))]
        _check(orc, n, w, g, bq, bk)
