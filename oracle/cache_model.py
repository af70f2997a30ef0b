"""Rolling-buffer KV cache model -- TEST INFRASTRUCTURE ONLY.

Cache layout (per batch entry and head) of ``g + w`` rows:
  * rows 0 .. g-1: sink rows; the token at position t < g is also kept in row t
    and never overwritten ("Sliding Window and Sparse Attention, from Longformer
    to CSA2", s2, attention sinks; "Local and Sparse Attention: Reading Fewer
    Token Positions", Figure 4 and the text after it: a position that is always
    read must stay stored after it leaves the window);
  * rows g .. g+w-1: the rolling buffer; position t overwrites slot t mod w,
    i.e. row g + (t mod w) (same s2, rolling buffer; Figure 4, circular
    overwrite).

``append`` writes tokens one by one in position order, which is the plain
meaning of a rolling buffer: a later token overwrites an earlier one in the
same slot.  ``logical_rows`` answers, for a query at position p, which stored
row holds each position the cache still has: ring slots hold the w most recent
positions; sink rows supply the sink positions that have left the window.  A
position that is in both is read once, from the ring.

Arrays are numpy or torch CPU tensors indexed [batch, head, row, d].
"""
from __future__ import annotations

import numpy as np


def ring_row(t: int, w: int, g: int) -> int:
    """Row of the rolling buffer that receives position t."""
    return g + (t % w)


def append(k_cache, v_cache, k_new, v_new, pos, w: int, g: int) -> None:
    """Write T new tokens per batch entry, token by token.

    k_new, v_new: [B, H, T, d]; pos[b]: position of token 0 of batch entry b.
    """
    B = k_new.shape[0]
    T = k_new.shape[2]
    for b in range(B):
        for t in range(T):
            P = int(pos[b]) + t
            r = ring_row(P, w, g)
            k_cache[b, :, r] = k_new[b, :, t]
            v_cache[b, :, r] = v_new[b, :, t]
            if P < g:
                k_cache[b, :, P] = k_new[b, :, t]
                v_cache[b, :, P] = v_new[b, :, t]


def logical_rows(p: int, w: int, g: int):
    """(positions, rows) the cache supplies for a query at position p.

    Only positions 0..p exist.  The ring holds the most recent min(p+1, w)
    positions; each earlier position below g comes from its sink row.
    """
    positions, rows = [], []
    for t in range(max(0, p - w + 1), p + 1):
        positions.append(t)
        rows.append(ring_row(t, w, g))
    for t in range(0, min(g, max(0, p - w + 1))):
        positions.append(t)
        rows.append(t)
    return np.asarray(positions, dtype=np.int64), np.asarray(rows, dtype=np.int64)
