"""Checks that pin the fp64 oracle to facts outside itself.

Each check takes an ``oracle.Oracle`` (the real build, or a copy with a
planted mistake) and returns a list of failure strings.  The facts used:

  * counts and read sets printed on "Local and Sparse Attention: Reading Fewer
    Token Positions" (Figures 1 and 2), stored under tests/golden/;
  * the dense additive-mask construction of "How does sliding window attention
    (SWA) reduce memory usage in long-context models?" (its Example: a lower
    triangle, then an upper triangle from diagonal -w+1, then -inf off the band),
    rebuilt here with torch.tril / torch.triu;
  * w >= n reduces to ordinary causal attention, which torch's
    scaled_dot_product_attention computes (fp64, CPU, is_causal=True);
  * closed forms: w = 1 gives O = V; constant V gives O = V; Q = 0 makes every
    attended logit equal up to the sink bias, so o_i is an explicit weighted
    mean over the attended keys;
  * a one-hot V with Q = 0 exposes the attended set as the nonzero pattern of
    O (a zeroed instead of -inf score would leak a positive weight);
  * the set-based brute force in ``oracle/brute.py`` on tiny inputs.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def golden_fig1():
    out = []
    for line in _rows("fig1_counts.txt"):
        vals = [int(x) for x in line.split()]
        n, w, g, total = vals[:4]
        out.append((n, w, g, total, vals[4:]))
    return out


def golden_fig2():
    out = []
    for line in _rows("fig2_read_sets.txt"):
        head, keys = line.split(":")
        n, w, g, i = (int(x) for x in head.split())
        out.append((n, w, g, i, [int(x) for x in keys.split()]))
    return out


def golden_fig4():
    out = []
    for line in _rows("fig4_ring.txt"):
        head, slots = line.split(":")
        w, g, last = (int(x) for x in head.split())
        out.append((w, g, last, [int(x) for x in slots.split()]))
    return out


def p5_dense_mask(n: int, w: int) -> np.ndarray:
    """The page's additive mask construction, 1 where the additive mask is 0."""
    causal = torch.tril(torch.ones(n, n))
    band = torch.triu(causal, diagonal=-w + 1)
    add = torch.full((n, n), float("-inf"))
    add[band == 1] = 0.0
    return (add == 0.0).numpy().astype(np.uint8)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def check_counts(orc):
    fails = []
    for n, w, g, total, per_row in golden_fig1():
        if orc.pair_count(n, w, g) != total:
            fails.append(f"pair_count({n},{w},{g}) != {total}")
        got = [orc.row_count(i, w, g) for i in range(n)]
        if got != per_row:
            fails.append(f"row counts ({n},{w},{g}) {got} != {per_row}")
    # No rule reads a future position (Figure 2 text): the grid is lower-triangular.
    for n, w, g in [(8, 3, 4), (6, 2, 6), (12, 5, 3)]:
        if np.any(np.triu(orc.mask(n, w, g), 1)):
            fails.append(f"mask({n},{w},{g}) reads a future position")
    for n, w, g, i, keys in golden_fig2():
        row = orc.mask(n, w, g)[i]
        if sorted(np.nonzero(row)[0].tolist()) != keys:
            fails.append(f"read set ({n},{w},{g}) row {i}: {np.nonzero(row)[0].tolist()} != {keys}")
    return fails


def check_p5_mask(orc):
    fails = []
    for n, w in [(6, 3), (8, 3), (9, 1), (7, 7), (5, 9), (33, 4)]:
        if not np.array_equal(orc.mask(n, w, 0), p5_dense_mask(n, w)):
            fails.append(f"mask({n},{w},0) differs from the tril/triu construction")
    return fails


def check_causal_sdpa(orc):
    fails = []
    for n, d, w, g in [(9, 4, 9, 0), (12, 8, 40, 3), (5, 2, 5, 5)]:
        q, k, v = (_rand((2, n, d), s) for s in (1, 2, 3))
        o, lse = orc.prefill(q, k, v, w=w, g=g, beta=0.0)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy()
        if np.max(np.abs(o - ref)) > 1e-12:
            fails.append(f"w>=n differs from causal SDPA (n={n}, w={w}, g={g})")
        scores = (tq @ tk.transpose(-1, -2)) / math.sqrt(d)
        scores = scores.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        ref_lse = torch.logsumexp(scores, dim=-1).numpy()
        if np.max(np.abs(lse - ref_lse)) > 1e-12:
            fails.append(f"w>=n lse differs from logsumexp (n={n})")
    return fails


def check_closed_forms(orc):
    fails = []
    # w = 1, no sinks: each query reads only itself, so o_i = v_i exactly.
    q, k, v = (_rand((11, 5), s) for s in (4, 5, 6))
    o, lse = orc.prefill(q, k, v, w=1, g=0)
    if not np.array_equal(o, v):
        fails.append("w=1 does not give O = V")
    s_diag = np.sum(q * k, axis=1) / math.sqrt(5)
    if np.max(np.abs(lse - s_diag)) > 1e-12:
        fails.append("w=1 lse is not the single scaled score")
    # constant V: any convex combination returns the constant.
    vc = np.full((11, 5), 0.375)
    o, _ = orc.prefill(q, k, vc, w=3, g=2, beta=1.5)
    if np.max(np.abs(o - 0.375)) > 1e-15:
        fails.append("constant V not reproduced")
    # Q = 0: logits are beta on sink keys, 0 elsewhere; o_i is the weighted mean
    # over window keys [max(0,i-w+1), i] and the sink keys below the window.
    n, d, w, g, beta = 14, 3, 4, 3, 4.0
    q0 = np.zeros((n, d))
    k, v = _rand((n, d), 7), _rand((n, d), 8)
    o, lse = orc.prefill(q0, k, v, w=w, g=g, beta=beta)
    for i in range(n):
        lo = max(0, i - w + 1)
        keys = list(range(lo, i + 1)) + list(range(0, min(g, lo)))
        wts = np.array([math.exp(beta) if j < g else 1.0 for j in keys])
        ref = (wts[:, None] * v[keys]).sum(0) / wts.sum()
        if np.max(np.abs(o[i] - ref)) > 1e-13:
            fails.append(f"Q=0 closed form row {i}")
            break
        if abs(lse[i] - math.log(wts.sum())) > 1e-13:
            fails.append(f"Q=0 lse row {i}")
            break
    return fails


def check_onehot(orc):
    """Q = 0, V[j, c] = [j == c]: O[i, j] > 0 exactly when key j is attended."""
    fails = []
    for n, w, g in [(8, 3, 0), (8, 3, 1), (10, 4, 2), (6, 7, 0)]:
        q = np.zeros((n, n))
        k = _rand((n, n), 9)
        v = np.eye(n)
        o, _ = orc.prefill(q, k, v, w=w, g=g, beta=0.0)
        pattern = (o != 0.0).astype(np.uint8)
        if not np.array_equal(pattern, orc.mask(n, w, g)):
            fails.append(f"one-hot pattern differs from the mask ({n},{w},{g})")
    return fails


def check_brute(orc, cases=None):
    from oracle import brute

    fails = []
    if cases is None:
        cases = [(7, 3, 2, 3, 0.7), (9, 1, 4, 2, -1.25), (6, 8, 0, 4, 0.0), (10, 4, 3, 3, 4.0)]
    for n, w, g, d, beta in cases:
        q, k, v = (_rand((n, d), 100 + s) for s in range(3))
        o, lse = orc.prefill(q, k, v, w=w, g=g, beta=beta)
        bo, blse = brute.attention(q.tolist(), k.tolist(), v.tolist(), w=w, g=g, beta=beta)
        if np.max(np.abs(o - np.array(bo))) > 1e-12 or np.max(np.abs(lse - np.array(blse))) > 1e-12:
            fails.append(f"brute force differs (n={n}, w={w}, g={g}, beta={beta})")
    return fails


ALL_CHECKS = [check_counts, check_p5_mask, check_causal_sdpa, check_closed_forms, check_onehot, check_brute]


def run_all(orc):
    fails = []
    for chk in ALL_CHECKS:
        try:
            fails += chk(orc)
        except Exception as e:  # a mutant may also crash or refuse
            fails.append(f"{chk.__name__} raised {e!r}")
    return fails
