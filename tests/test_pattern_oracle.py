"""The oracle's dilated and landmark patterns against facts outside it (CPU).

Pins: the read sets printed with Figure 2 of "Local and Sparse Attention:
Reading Fewer Token Positions" (q7 reads {0, 5, 6, 7} with the first
position as anchor, {0, 4, 5, 6, 7} with landmarks every 4; p3 cannot read
p4); reductions to the dense window oracle (a dilation of 1 is the window;
landmarks every position are full causal attention; landmarks further apart
than the sequence leave the window plus position 0, i.e. one sink); a
dilated window equals the plain window over each strided residue class; the
closed-form read count min(w, floor(i/r)+1) of a dilated window.
"""
import numpy as np
import pytest

from oracle import patterns


def test_figure2_read_sets():
    assert patterns.read_set(7, "landmark", w=3, g=0, r=4) == {0, 4, 5, 6, 7}
    assert patterns.read_set(7, "window", w=3, g=1) == {0, 5, 6, 7}
    assert 4 not in patterns.read_set(3, "landmark", w=3, g=0, r=4)
    assert patterns.read_set(4, "landmark", w=3, g=0, r=4) == {0, 2, 3, 4}


def test_dilated_counts():
    for w, r in [(3, 2), (5, 4), (1, 3), (8, 1)]:
        for i in range(60):
            assert len(patterns.read_set(i, "dilated", w, r=r)) == min(w, i // r + 1)


def _qkv(n, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))


@pytest.mark.parametrize("n,w", [(40, 7), (64, 64), (50, 1)])
def test_reductions_to_window_oracle(orc, n, w):
    q, k, v = _qkv(n, 16, n + w)
    ro, rl = orc.prefill(q, k, v, w=w, g=0)
    o, l = patterns.prefill(q, k, v, "dilated", w=w, r=1)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(l, rl, atol=1e-12)
    # landmarks at every position: full causal attention
    ro, rl = orc.prefill(q, k, v, w=n, g=0)
    o, l = patterns.prefill(q, k, v, "landmark", w=w, g=0, r=1)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    # landmarks further apart than the sequence: window plus position 0 = one sink
    ro, rl = orc.prefill(q, k, v, w=w, g=1, beta=0.0)
    o, l = patterns.prefill(q, k, v, "landmark", w=w, g=0, r=n + 5)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(l, rl, atol=1e-12)


@pytest.mark.parametrize("n,w,r", [(45, 4, 3), (64, 8, 4), (30, 30, 7)])
def test_dilated_is_window_over_residue_classes(orc, n, w, r):
    q, k, v = _qkv(n, 8, 7 * n + r)
    o, l = patterns.prefill(q, k, v, "dilated", w=w, r=r)
    for c in range(r):
        ro, rl = orc.prefill(q[c::r], k[c::r], v[c::r], w=w, g=0)
        np.testing.assert_allclose(o[c::r], ro, atol=1e-12)
        np.testing.assert_allclose(l[c::r], rl, atol=1e-12)


def test_landmark_sinks_and_bias(orc):
    # with g sinks and bias, landmarks further apart than n: equals window + sinks + bias
    n, w, g, beta = 50, 6, 3, 1.5
    q, k, v = _qkv(n, 8, 11)
    ro, rl = orc.prefill(q, k, v, w=w, g=g, beta=beta)
    o, l = patterns.prefill(q, k, v, "landmark", w=w, g=g, r=1000, beta=beta)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(l, rl, atol=1e-12)
