"""Grouped-query attention in the fp64 oracle, pinned to closed forms (CPU only).

Source: "Sliding Window and Sparse Attention, from Longformer to CSA2", s10
glossary, GQA (several query heads share one key/value head).  The page does
not say which query heads share a key/value head; the reading taken is
consecutive groups.  The pins:

  * the head map itself for multi-head (identity), multi-query (all 0) and
    two groups of four;
  * a constant value row c_j in key/value head j makes every attended output
    of a query head equal c_j of its own key/value head, whatever the weights;
  * zero keys in key/value head j make every weight of the window equal, so a
    query head of that group outputs the plain mean of its attended values;
    heads of the other groups see random keys and do not;
  * one key/value head per query head reduces to the multi-head oracle.
"""
import numpy as np
import pytest

import oracle


def test_head_map_table():
    assert [oracle.kv_head_of(h, 8, 8) for h in range(8)] == list(range(8))
    assert [oracle.kv_head_of(h, 8, 1) for h in range(8)] == [0] * 8
    assert [oracle.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 8, 3)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("kv_heads", [1, 2, 4, 8])
def test_constant_values_follow_the_group(orc, kv_heads):
    B, H, n, d, w, g = 2, 8, 24, 16, 5, 2
    q, k = _rand((B, H, n, d), 1), _rand((B, kv_heads, n, d), 2)
    c = _rand((B, kv_heads, d), 3)
    v = np.broadcast_to(c[:, :, None, :], (B, kv_heads, n, d)).copy()
    o, _ = orc.prefill(q, k, v, w=w, g=g, beta=0.7)
    G = H // kv_heads
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(o[b, h], np.broadcast_to(c[b, h // G], (n, d)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("kv_heads", [2, 4])
def test_zero_keys_give_window_means(orc, kv_heads):
    B, H, n, d, w = 1, 8, 20, 8, 6
    q, v = _rand((B, H, n, d), 4), _rand((B, kv_heads, n, d), 5)
    k = _rand((B, kv_heads, n, d), 6)
    k[:, 0::2] = 0.0  # even key/value heads: every score is 0
    o, _ = orc.prefill(q, k, v, w=w, g=0)
    G = H // kv_heads
    for h in range(H):
        j = h // G
        mean = np.stack([v[0, j, max(0, i - w + 1): i + 1].mean(axis=0) for i in range(n)])
        err = np.max(np.abs(o[0, h] - mean))
        if j % 2 == 0:
            assert err < 1e-12, (h, j, err)
        else:
            assert err > 1e-3, (h, j, err)


def test_one_kv_head_per_query_head_is_multi_head(orc):
    q, k, v = _rand((1, 4, 16, 8), 7), _rand((1, 4, 16, 8), 8), _rand((1, 4, 16, 8), 9)
    o1, l1 = orc.prefill(q, k, v, w=4, g=1, beta=-0.3)
    o2, l2 = orc.prefill(q, oracle.expand_kv_heads(4, k), oracle.expand_kv_heads(4, v), w=4, g=1, beta=-0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_expand_rejects_non_divisor():
    with pytest.raises(ValueError):
        oracle.expand_kv_heads(6, np.zeros((1, 4, 2, 2)))
