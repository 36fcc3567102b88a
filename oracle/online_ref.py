"""The online-softmax recurrence in float64, over arbitrary key tilings.

TEST INFRASTRUCTURE ONLY (same rules as ``attention_ref``: tests, the smoke
check and the benchmark's CPU leg may use it; the product never does).

The method (page "22. GPU Engineering: Correctness, Throughput, and
Attention", sec. 22.5; page "GPU Programming & Kernel Development",
Self-check): each query row carries a state -- the largest score seen so far
``m``, the normaliser ``l`` of the weights taken relative to ``m`` and the
weighted sum of value rows ``o`` relative to the same reference -- starting
from (-inf, 0, 0).  A tile of scores S moves the reference to
m' = max(m, max S); the old state is rescaled by exp(m - m'), the tile's
weights are exp(S - m'), and both are added in.  After the last tile the row's
output is o / l and its log-normaliser m + ln l.  Hidden keys (future keys
under the causal rule of sec. 22.7) score -inf before the maximum and the sum.
While a row has seen no visible key its reference would be -inf; the lab of
sec. 22.7 then uses 0 as exponent reference so that -inf - (-inf) never
occurs, and a row that ends with l = 0 gets output 0 and log-normaliser -inf.

This harness states the recurrence row by row, one scalar state per query,
so that it can be read against the equations above; its only purpose is to
pin the recurrence against the two-pass definition in ``attention_ref``
under every way of cutting the key axis into tiles (the property the GPU
kernel relies on).  It is deliberately slow.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["online_attention_ref", "uniform_bounds", "all_compositions"]


def uniform_bounds(nk: int, tile: int):
    """Tile boundaries [0, t, 2t, ..., nk] for a uniform tile width."""
    if tile < 1:
        raise ValueError("tile must be positive")
    b = list(range(0, nk, tile)) + [nk]
    return b if b[0] == 0 and nk > 0 else [0, nk]


def all_compositions(nk: int):
    """Every way to cut keys 0..nk-1 into consecutive non-empty tiles.

    Yields boundary lists [0, c1, ..., nk]; there are 2**(nk-1) of them.
    """
    for mask in range(1 << max(nk - 1, 0)):
        cuts = [c + 1 for c in range(nk - 1) if mask >> c & 1]
        yield [0] + cuts + [nk]


class _RowState:
    """(m, l, o) of one query row under the sec. 22.5 update."""

    def __init__(self, width: int):
        self.m = -math.inf
        self.l = 0.0
        self.o = np.zeros(width)

    def absorb(self, scores, values):
        """One tile: ``scores`` (hidden keys at -inf) and their value rows."""
        m_next = max(self.m, max(scores, default=-math.inf))
        reference = m_next if m_next != -math.inf else 0.0      # sec. 22.7 safe reference
        keep = math.exp(self.m - reference)                      # exp(m - m') for the old state
        weights = np.array([math.exp(s - reference) for s in scores])
        self.l = keep * self.l + float(weights.sum())
        self.o = keep * self.o + weights @ values
        self.m = m_next

    def result(self):
        """(output row, log-normaliser); a row that saw no key gives (0, -inf)."""
        if self.l > 0.0:
            return self.o / self.l, self.m + math.log(self.l)
        return np.zeros_like(self.o), -math.inf


def online_attention_ref(q, k, v, scale: float, bounds, causal: bool = False,
                         query_offset: int = 0, trace=None):
    """Run the online update tile by tile; return (O, LSE) like attention_ref.

    bounds: increasing key boundaries [0, b1, ..., nk]; tile t holds keys
            bounds[t] .. bounds[t+1]-1.
    trace:  optional list; after the run it receives, for each tile t in
            order, (m, l) -- arrays over the query rows of the state after
            tile t -- so a test can inspect the running state.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    if list(bounds[:1]) != [0] or bounds[-1] != nk or any(
            b1 <= b0 for b0, b1 in zip(bounds[:-1], bounds[1:])):
        raise ValueError("bounds must rise strictly from 0 to nk")
    tiles = list(zip(bounds[:-1], bounds[1:]))

    out = np.zeros((nq, v.shape[1]))
    lse = np.full(nq, -math.inf)
    m_after = np.zeros((len(tiles), nq))
    l_after = np.zeros((len(tiles), nq))
    for i in range(nq):
        position = i + query_offset                 # the row's absolute position
        state = _RowState(v.shape[1])
        for t, (first, end) in enumerate(tiles):
            scores = []
            for j in range(first, end):
                hidden = causal and j > position
                scores.append(-math.inf if hidden else float(scale) * float(q[i] @ k[j]))
            state.absorb(scores, v[first:end])
            m_after[t, i], l_after[t, i] = state.m, state.l
        out[i], lse[i] = state.result()
    if trace is not None:
        trace.extend((m_after[t].copy(), l_after[t].copy()) for t in range(len(tiles)))
    return out, lse
