"""A model of the online-softmax recurrence in float64, one key tile at a time.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages describe the running state a query row carries across key/value
tiles: the largest score seen so far, the sum of the exponentials taken
relative to it, and the value rows weighted by those exponentials ("Flash
Attention, tiled: exact attention without the T x T HBM matrix", sections
"What happens when the maximum changes" and "From the example to tiled GPU
work"; "FlashAttention: the IO-aware Attention Kernel", section 3.2).  This
model writes that state as a summary of a SET of keys:

    State(keys) = (m, l, o) with m = max score over the keys,
                  l = sum of exp(score - m),  o = sum of exp(score - m) * v.

Two summaries of disjoint key sets merge exactly: bring both to the larger
maximum (multiply each l and o by exp(its m - larger m)) and add.  Folding a
tile into a row is then "summarise the tile on its own, merge it into the
row", and merging the summaries of key splits is the combine step of
"FlashAttention and Fused Kernels: Attention Without the n x n Matrix", Step 4.
The empty set is (-inf, 0, 0) and is the identity of the merge.  The row's
output is o / l and its log-sum-exp m + ln l.
"""
from __future__ import annotations

import math

import numpy as np


class RowState:
    """The (m, l, o) summary of the keys a query row has seen so far."""

    def __init__(self, d: int):
        self.m = -math.inf
        self.l = 0.0
        self.o = np.zeros(d, dtype=np.float64)

    @classmethod
    def of_tile(cls, s_tile: np.ndarray, v_tile: np.ndarray) -> "RowState":
        """The summary of one tile alone: its own maximum, sum and weighted values."""
        s_tile = np.asarray(s_tile, dtype=np.float64)
        v_tile = np.asarray(v_tile, dtype=np.float64)
        st = cls(v_tile.shape[1])
        if s_tile.size:
            st.m = float(np.max(s_tile))
            w = np.exp(s_tile - st.m)
            st.l = float(np.sum(w))
            st.o = w @ v_tile
        return st

    def merge(self, other: "RowState") -> None:
        """Absorb the summary of a disjoint key set."""
        if other.l == 0.0:
            return
        if self.l == 0.0:
            self.m, self.l, self.o = other.m, other.l, other.o.copy()
            return
        top = max(self.m, other.m)
        a, b = math.exp(self.m - top), math.exp(other.m - top)
        self.l = a * self.l + b * other.l
        self.o = a * self.o + b * other.o
        self.m = top

    def update(self, s_tile: np.ndarray, v_tile: np.ndarray) -> None:
        """Fold one tile of scores (length n) and its value rows (n x d) into the row."""
        self.merge(RowState.of_tile(s_tile, v_tile))

    def output(self) -> np.ndarray:
        return self.o / self.l

    def lse(self) -> float:
        return self.m + math.log(self.l)


def combine(states):
    """Merge the summaries of disjoint key ranges (for example, key splits) of one row."""
    out = RowState(states[0].o.shape[0])
    for s in states:
        out.merge(s)
    return out


def attention_online_f64(q, k, v, causal: bool, scale: float, block: int):
    """Tiled online-softmax attention over (B, H, T, d) float64 arrays.

    Keys are visited in tiles of ``block``; each row keeps its own summary.
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
