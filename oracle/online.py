"""The online-softmax recurrence, tile by tile, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This follows the row-local update stated on "Flash Attention, tiled: exact
attention without the T x T HBM matrix", section "What happens when the maximum
changes", and the same recurrence written as equations on "FlashAttention: the
IO-aware Attention Kernel", section 3.2 (Online softmax):

    m' = max(m, max(s_tile))
    r  = exp(m - m')                (taken as 0 while m is still -inf)
    p  = exp(s_tile - m')
    l  = r * l + sum(p)
    o  = r * o + p^T @ V_tile
    m  = m'

and, after the last tile, Y = o / l.  The state (m, l, o) belongs to one query
row, starts at (-inf, 0, 0) and is never reset between key/value tiles
("From the example to tiled GPU work").

The partial-state merge in ``combine`` is the Flash-Decoding combine of
"FlashAttention and Fused Kernels: Attention Without the n x n Matrix", Step 4:
each split gives a partial state and the pieces are rescaled to the larger
maximum and added.
"""
from __future__ import annotations

import math

import numpy as np


class RowState:
    """Running (m, l, o) for one query row."""

    def __init__(self, d: int):
        self.m = -math.inf
        self.l = 0.0
        self.o = np.zeros(d, dtype=np.float64)

    def update(self, s_tile: np.ndarray, v_tile: np.ndarray) -> None:
        """Fold one tile of scores (len n) and its values (n x d) into the state."""
        s_tile = np.asarray(s_tile, dtype=np.float64)
        v_tile = np.asarray(v_tile, dtype=np.float64)
        if s_tile.size == 0:
            return
        m_new = max(self.m, float(np.max(s_tile)))
        r = 0.0 if self.m == -math.inf else math.exp(self.m - m_new)
        p = np.exp(s_tile - m_new)
        self.l = r * self.l + float(np.sum(p))
        self.o = r * self.o + p @ v_tile
        self.m = m_new

    def output(self) -> np.ndarray:
        return self.o / self.l

    def lse(self) -> float:
        return self.m + math.log(self.l)


def combine(states):
    """Merge partial row states computed on disjoint key ranges."""
    states = [s for s in states if s.l > 0.0]
    out = RowState(states[0].o.shape[0])
    m = max(s.m for s in states)
    out.m = m
    out.l = sum(math.exp(s.m - m) * s.l for s in states)
    out.o = sum(math.exp(s.m - m) * s.o for s in states)
    return out


def attention_online_f64(q, k, v, causal: bool, scale: float, block: int):
    """Tiled online-softmax attention over (B, H, T, d) float64 arrays.

    Keys are visited in tiles of ``block``; each row keeps its own state.
    Returns ``(o, lse)`` like the plain oracle.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for i in range(T):
                st = RowState(d)
                n_vis = i + 1 if causal else T
                for start in range(0, n_vis, block):
                    stop = min(start + block, n_vis)
                    s = scale * (k[b, h, start:stop] @ q[b, h, i])
                    st.update(s, v[b, h, start:stop])
                o[b, h, i] = st.output()
                lse[b, h, i] = st.lse()
    return o, lse
