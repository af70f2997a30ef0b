"""The oracle's log-sum-exp merge against direct softmaxes (CPU only).

Pins: a softmax over a key set split into two disjoint parts equals the
merge of the two partial softmaxes (brute force over explicit scores); an
empty part (lse = -inf) leaves the other part unchanged; merging a part with
itself keeps o and adds ln 2 to lse; the merge is symmetric.
"""
import math

import numpy as np

import oracle


def _partial(scores, values):
    """softmax(scores) @ values and log-sum-exp of scores (empty: 0, -inf)."""
    if scores.size == 0:
        return np.zeros(values.shape[-1]), -math.inf
    m = scores.max()
    e = np.exp(scores - m)
    return e @ values / e.sum(), m + math.log(e.sum())


def test_split_softmax_merges_to_union():
    rng = np.random.default_rng(3)
    for trial in range(50):
        nk, d = int(rng.integers(1, 40)), 8
        s = rng.standard_normal(nk) * rng.uniform(0.1, 20.0)
        v = rng.standard_normal((nk, d))
        cut = rng.permutation(nk)
        k = int(rng.integers(0, nk + 1))
        a, b = np.sort(cut[:k]), np.sort(cut[k:])
        oa, la = _partial(s[a], v[a])
        ob, lb = _partial(s[b], v[b])
        ou, lu = _partial(s, v)
        o, lse = oracle.lse_merge(oa[None], np.array([la]), ob[None], np.array([lb]))
        np.testing.assert_allclose(o[0], ou, rtol=0, atol=1e-12)
        assert abs(lse[0] - lu) < 1e-12


def test_empty_part_and_self_merge():
    rng = np.random.default_rng(4)
    o1, l1 = rng.standard_normal((5, 4)), rng.standard_normal(5)
    ninf = np.full(5, -np.inf)
    o, lse = oracle.lse_merge(o1, l1, np.zeros((5, 4)), ninf)
    assert np.array_equal(o, o1) and np.array_equal(lse, l1)
    o, lse = oracle.lse_merge(np.zeros((5, 4)), ninf, o1, l1)
    assert np.array_equal(o, o1) and np.array_equal(lse, l1)
    o, lse = oracle.lse_merge(o1, l1, o1, l1)
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(lse, l1 + math.log(2.0), atol=1e-15)
    o, lse = oracle.lse_merge(np.zeros((5, 4)), ninf, np.zeros((5, 4)), ninf)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_merge_is_symmetric():
    rng = np.random.default_rng(5)
    oa, ob = rng.standard_normal((7, 3)), rng.standard_normal((7, 3))
    la, lb = rng.standard_normal(7) * 5, rng.standard_normal(7) * 5
    o1, l1 = oracle.lse_merge(oa, la, ob, lb)
    o2, l2 = oracle.lse_merge(ob, lb, oa, la)
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    np.testing.assert_allclose(l1, l2, atol=1e-15)
