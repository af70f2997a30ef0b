"""The fp64 oracle against facts outside itself (CPU only).

Also plants plausible mistakes in copies of the oracle's C source and checks
that every one of them is caught by at least one pin.
"""
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import brute
from tests import oracle_pins as pins


def test_pins_hold(orc):
    assert pins.run_all(orc) == []


@pytest.mark.parametrize(
    "n,w,g,expected",
    [
        (8, 3, 0, 21),      # printed: page "Local and Sparse Attention ...", Figure 1
        (8, 8, 0, 36),      # printed: same figure, full causal
        (8, 30, 0, 36),     # w > n is full causal too
        (6, 3, 0, 15),      # the 6 x 3 additive mask of the SWA Q&A page's example
        (8, 3, 1, 26),      # Figure 2 anchor rule added to Figure 1's window
        (256, 64, 0, 14368),  # tiny fp32 workload: n*w - w(w-1)/2
    ],
)
def test_pair_counts(orc, n, w, g, expected):
    assert orc.pair_count(n, w, g) == expected


def closed_form_pairs(n, w, g):
    """Row i reads min(i+1, w) window keys plus the sink keys below the window,
    min(g, max(0, i-w+1)); summed in closed form where possible."""
    total = 0
    for i in range(n):
        total += min(i + 1, w) + min(g, max(0, i - w + 1))
    return total


@pytest.mark.parametrize("n,w,g", [(1, 1, 0), (40, 7, 5), (100, 100, 3), (257, 64, 4), (300, 1, 2), (16, 3, 20)])
def test_pair_count_matches_row_formula(orc, n, w, g):
    assert orc.pair_count(n, w, g) == closed_form_pairs(n, w, g)
    if g == 0 and w <= n:
        assert orc.pair_count(n, w, g) == n * w - w * (w - 1) // 2


def test_large_config_pair_counts(orc):
    # Mistral-7B-shaped prefill (n=16384, w=4096) and the sink config
    # (n=32768, w=4096, g=4): exact attended pairs per head.
    assert orc.pair_count(16384, 4096, 0) == 16384 * 4096 - 4096 * 4095 // 2 == 58_722_304
    assert orc.pair_count(32768, 4096, 4) == closed_form_pairs(32768, 4096, 4) == 125_945_850


def test_brute_force_sweep(orc):
    """Set-based brute force vs the C oracle over many tiny (n, w, g)."""
    rng = np.random.default_rng(0)
    d = 3
    for n in (1, 2, 3, 5, 8, 13, 21):
        for w in range(1, n + 3):
            for g in range(0, n + 2):
                beta = float(rng.choice([0.0, 4.0, -2.5]))
                q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
                o, lse = orc.prefill(q, k, v, w=w, g=g, beta=beta)
                bo, blse = brute.attention(q.tolist(), k.tolist(), v.tolist(), w=w, g=g, beta=beta)
                assert np.max(np.abs(o - np.array(bo))) <= 1e-12, (n, w, g)
                assert np.max(np.abs(lse - np.array(blse))) <= 1e-12, (n, w, g)
                m = orc.mask(n, w, g)
                for i in range(n):
                    assert set(np.nonzero(m[i])[0].tolist()) == brute.attended_set(i, w, g)


def test_brute_force_n40(orc):
    rng = np.random.default_rng(1)
    n, d = 40, 4
    for w, g in [(1, 0), (5, 4), (39, 1), (40, 0), (42, 41), (17, 0)]:
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        o, lse = orc.prefill(q, k, v, w=w, g=g, beta=1.0)
        bo, blse = brute.attention(q.tolist(), k.tolist(), v.tolist(), w=w, g=g, beta=1.0)
        assert np.max(np.abs(o - np.array(bo))) <= 1e-12
        assert np.max(np.abs(lse - np.array(blse))) <= 1e-12


def test_rows_subset_and_batch(orc):
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((2, 3, 30, 8)) for _ in range(3))
    o_all, lse_all = orc.prefill(q, k, v, w=6, g=2, beta=0.5)
    rows = [29, 0, 7, 6]
    o_s, lse_s = orc.prefill(q, k, v, w=6, g=2, beta=0.5, rows=rows)
    assert o_all.shape == (2, 3, 30, 8)
    assert np.array_equal(o_s, o_all[:, :, rows])
    assert np.array_equal(lse_s, lse_all[:, :, rows])


def test_rows_sum_to_one_and_bounded(orc):
    """Outputs are convex combinations: with V in [0,1] every output is in [0,1]."""
    rng = np.random.default_rng(3)
    n, d = 50, 6
    q, k = rng.standard_normal((n, d)) * 3, rng.standard_normal((n, d)) * 3
    v = rng.random((n, d))
    o, _ = orc.prefill(q, k, v, w=9, g=4, beta=4.0)
    assert np.all(o >= -1e-15) and np.all(o <= 1 + 1e-15)


def test_decode_refuses_incomplete_or_duplicate_rows(orc):
    d, w, g, p = 4, 5, 2, 20
    rng = np.random.default_rng(4)
    pos = list(range(p - w + 1, p + 1)) + [0, 1]
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, len(pos), d))
    v = rng.standard_normal((1, len(pos), d))
    orc.decode(q, [p], [pos], k, v, w=w, g=g)
    with pytest.raises(ValueError):
        orc.decode(q, [p], [pos[:-1] + [-1]], k, v, w=w, g=g)   # sink 1 missing
    with pytest.raises(ValueError):
        orc.decode(q, [p], [pos[:-1] + [0]], k, v, w=w, g=g)    # sink 0 twice


# --- planted mistakes --------------------------------------------------------
# Each entry replaces one fragment of the oracle's C source; the pins must
# reject every resulting oracle.
MUTANTS = {
    "window one too wide": ("if (j >= i - w + 1) return 1;", "if (j >= i - w) return 1;"),
    "window one too narrow": ("if (j >= i - w + 1) return 1;", "if (j > i - w + 1) return 1;"),
    "sinks read from the future": ("if (j < 0 || j > i) return 0;", "if (j < 0 || (j > i && j >= g)) return 0;"),
    "no sinks": ("if (j < g) return 1;", "if (j < 0) return 1;"),
    "masked score zeroed, not -inf": ("s[t] = -INFINITY;", "s[t] = 0.0;"),
    "scale dropped": ("s[t] = scale * dot(", "s[t] = dot("),
    "sink bias on every key": ("(j < g ? beta : 0.0)", "beta"),
    "sink bias only outside the window": ("(j < g ? beta : 0.0)", "((j < g && j < i - w + 1) ? beta : 0.0)"),
    "values and keys swapped": ("const double *vt = vrow + t * d;", "const double *vt = krow + t * d;"),
    "normaliser dropped": ("o[c] /= l;", "o[c] /= 1.0;"),
    "lse without the max": ("*lse = m + log(l);", "*lse = log(l);"),
    "dot product index": ("s += a[c] * b[c];", "s += a[c] * b[0];"),
    "sign of the score": ("s[t] = scale * dot(", "s[t] = -scale * dot("),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new)
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", str(so), str(c)])
    fails = pins.run_all(oracle.Oracle(str(so)))
    assert fails, f"planted mistake '{name}' passed every pin"
