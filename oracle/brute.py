"""Set-based brute force for tiny inputs -- TEST INFRASTRUCTURE ONLY.

A second evaluation of the same definition, built differently from the C
oracle so that the two can check each other:

  * the attended set is the Python ``set`` union of the window
    {max(0, i-w+1), ..., i} and the sink positions {0, ..., min(g, i+1)-1};
    a position in both is one element of the set ("Local and Sparse
    Attention: Reading Fewer Token Positions", Figure 2 and its text);
  * only positions in the set are scored (no -inf entries at all);
  * sums are exactly rounded with ``math.fsum``.

Scaled dot-product attention and the LSE follow "Sliding Window and Sparse
Attention, from Longformer to CSA2", s1 and the s10 glossary.
"""
from __future__ import annotations

import math


def attended_set(i: int, w: int, g: int) -> set[int]:
    window = set(range(max(0, i - w + 1), i + 1))
    sinks = set(range(0, min(g, i + 1)))
    return window | sinks


def attention(q, k, v, w: int, g: int = 0, scale: float | None = None, beta: float = 0.0):
    """q, k, v: lists (or arrays) of n rows of d floats.  Returns (o, lse)."""
    n = len(q)
    d = len(q[0]) if n else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs, lses = [], []
    for i in range(n):
        keys = sorted(attended_set(i, w, g))
        scores = []
        for j in keys:
            s = scale * math.fsum(float(q[i][c]) * float(k[j][c]) for c in range(d))
            if j < g:
                s += beta
            scores.append(s)
        m = max(scores)
        e = [math.exp(s - m) for s in scores]
        l = math.fsum(e)
        o = [math.fsum(e[t] * float(v[j][c]) for t, j in enumerate(keys)) / l for c in range(d)]
        outs.append(o)
        lses.append(m + math.log(l))
    return outs, lses
