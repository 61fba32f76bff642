"""fp64 model of the online-softmax recurrence, one query row at a time.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg import it; it shares no code with the HIP library.

It follows the steps the pages give for one query row whose keys arrive tile
by tile (kgptalkie "Flash Attention: Why Memory Traffic, Not Compute, Is the
Bottleneck", sections "Softmax Looks Like an Obstacle" and "Carry the Actual
Values Through Both Tiles"; aimlrounds "FlashAttention", section "Softmax
without seeing the whole row"):
  state (m, l, u): the largest score so far, the sum of exponentials taken
  relative to m, and the value-weighted sum of those exponentials;
  on a tile with maximum m_t: m' = max(m, m_t); both l and u are multiplied
  by e^(m - m') before the tile's own terms e^(s - m') are added;
  the output is u / l.
Merging two partial states of disjoint key sets uses the same rescale rule
(split-KV decoding, aimlrounds page, table "FlashAttention 1, 2, 3" note on
FlashDecoding).

The tests use it to show that the recurrence reproduces the pages' worked
rows and equals the three-step oracle for every tile size.
"""
from __future__ import annotations

import math

import numpy as np


class RowState:
    """Running (m, l, u) of one query row; u has the width of a value row."""

    def __init__(self, width: int):
        self.m = -math.inf
        self.l = 0.0
        self.u = np.zeros(width)

    def absorb(self, scores: np.ndarray, values: np.ndarray) -> None:
        """Fold in one tile: scores [n] (already scaled), values [n, width]."""
        if scores.size == 0:
            return
        m_new = max(self.m, float(np.max(scores)))
        alpha = math.exp(self.m - m_new) if self.m != -math.inf else 0.0
        w = np.exp(scores - m_new)
        self.l = alpha * self.l + float(np.sum(w))
        self.u = alpha * self.u + w @ values
        self.m = m_new

    def output(self) -> np.ndarray:
        return self.u / self.l if self.l > 0 else np.zeros_like(self.u)

    def lse(self) -> float:
        return self.m + math.log(self.l) if self.l > 0 else -math.inf


def merge(states) -> RowState:
    """Combine partial states over disjoint key sets into one."""
    states = [s for s in states if s.l > 0]
    width = states[0].u.shape[0] if states else 0
    out = RowState(width)
    if not states:
        return out
    m = max(s.m for s in states)
    out.m = m
    out.l = sum(math.exp(s.m - m) * s.l for s in states)
    out.u = sum(math.exp(s.m - m) * s.u for s in states)
    return out


def row_tiles(scores, values, tile: int):
    """Run one row through the recurrence with tiles of `tile` keys.

    Returns the list of states after each tile (copies), last one final."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if values.ndim == 1:
        values = values[:, None]
    st = RowState(values.shape[1])
    history = []
    for j0 in range(0, scores.shape[0], tile):
        st.absorb(scores[j0:j0 + tile], values[j0:j0 + tile])
        snap = RowState(values.shape[1])
        snap.m, snap.l, snap.u = st.m, st.l, st.u.copy()
        history.append(snap)
    return history


def attention_online(q, k, v, scale: float, causal: bool, tile: int):
    """Tiled attention for one head: q [Tq,d], k and v [Tk,d], keys in tiles.

    Returns O [Tq,d] and LSE [Tq]; masked keys are dropped before a tile is
    absorbed (causal, diagonal aligned bottom-right)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Tk = q.shape[0], k.shape[0]
    o = np.zeros((Tq, v.shape[1]))
    lse = np.zeros(Tq)
    for i in range(Tq):
        last = Tk - 1 if not causal else i + (Tk - Tq)
        st = RowState(v.shape[1])
        for j0 in range(0, Tk, tile):
            j1 = min(Tk, j0 + tile, last + 1)
            if j1 <= j0:
                break
            st.absorb(scale * (k[j0:j1] @ q[i]), v[j0:j1])
        o[i] = st.output()
        lse[i] = st.lse()
    return o, lse
