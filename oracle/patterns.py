"""Fixed sparse patterns beyond the window: dilated windows and landmarks.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH (see ``oracle/__init__``).

Sources:
  * "Sliding Window and Sparse Attention, from Longformer to CSA2", s2
    (dilated windows: every r-th key of a wider band, the cost of a window
    of w) and s4 (any fixed pattern as block-sparse tiles);
  * "Local and Sparse Attention: Reading Fewer Token Positions", Figure 2
    and its text (landmarks at regular intervals added to the latest
    positions, each position read once, never the future).
Readings (the pages leave these open): a dilated window of w reads the w
positions i, i-r, ..., i-(w-1)r that exist (no sinks); the landmark rule
reads the window i-w+1 .. i, the sinks 0 .. g-1 and every position j <= i
with j mod r == 0, each once, with the sink bias on positions < g.

``read_set`` is the set definition; ``prefill`` evaluates dense fp64 rows
over it (a plain masked softmax, numpy), for sizes where O(n^2) is cheap.
"""
from __future__ import annotations

import math

import numpy as np


def read_set(i: int, kind: str, w: int, g: int = 0, r: int = 1) -> set[int]:
    """Positions query i reads under pattern kind ("window", "dilated", "landmark")."""
    if kind == "dilated":
        return {i - k * r for k in range(w) if i - k * r >= 0}
    s = set(range(max(0, i - w + 1), i + 1)) | set(range(min(g, i + 1)))
    if kind == "landmark":
        s |= {j for j in range(0, i + 1, r)}
    elif kind != "window":
        raise ValueError(kind)
    return s


def prefill(q, k, v, kind: str, w: int, g: int = 0, r: int = 1, scale: float | None = None, beta: float = 0.0,
            rows=None):
    """q, k, v: [n, d] (one head; K/V already matched to the query head).
    Returns (o [nrows, d], lse [nrows]) in fp64."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    n, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    bias = np.where(np.arange(n) < g, beta, 0.0)
    for t, i in enumerate(rows):
        js = np.array(sorted(read_set(int(i), kind, w, g, r)), dtype=np.int64)
        s = scale * (k[js] @ q[i]) + bias[js]
        m = s.max()
        e = np.exp(s - m)
        o[t] = e @ v[js] / e.sum()
        lse[t] = m + math.log(e.sum())
    return o, lse
