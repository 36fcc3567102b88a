"""The online-softmax recurrence in float64, over arbitrary key tilings.

TEST INFRASTRUCTURE ONLY (same rules as ``attention_ref``: tests, the smoke
check and the benchmark's CPU leg may use it; the product never does).

This harness states the method itself -- page "22. GPU Engineering:
Correctness, Throughput, and Attention", sec. 22.5 (the running max ``m``,
normaliser ``l`` and unnormalised accumulator ``o``, started at -inf, 0, 0 and
updated once per score tile) and the worked lab of sec. 22.7 (a still fully
hidden row uses 0 as its exponent reference, so that -inf minus -inf never
occurs; a row that never sees a key ends with output 0 and LSE -inf).  Page
"GPU Programming & Kernel Development" (Self-check) states the same rescale by
exp(m_old - m_new) and the final division by l.

Its purpose is to pin the recurrence against the two-pass definition in
``attention_ref``: under every way of cutting the key axis into tiles the two
must agree to float64 rounding, which is the property the GPU kernel relies
on.  It is deliberately slow and literal.
"""
from __future__ import annotations

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


def online_attention_ref(q, k, v, scale: float, bounds, causal: bool = False,
                         query_offset: int = 0, trace=None):
    """Run the online update tile by tile; return (O, LSE) like attention_ref.

    bounds: increasing key boundaries [0, b1, ..., nk]; tile t holds keys
            bounds[t] .. bounds[t+1]-1.
    trace:  optional list; after each tile, (m.copy(), l.copy()) is appended
            so a test can inspect the running state.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    if list(bounds[:1]) != [0] or bounds[-1] != nk or any(
            b1 <= b0 for b0, b1 in zip(bounds[:-1], bounds[1:])):
        raise ValueError("bounds must rise strictly from 0 to nk")

    m = np.full(nq, -np.inf)                    # running maximum
    l = np.zeros(nq)                            # running normaliser
    o = np.zeros((nq, v.shape[1]))              # unnormalised weighted values
    qpos = np.arange(nq) + query_offset

    for lo, hi in zip(bounds[:-1], bounds[1:]):
        S = scale * (q @ k[lo:hi].T)            # one score tile
        if causal:                              # hide future keys before max/sum
            S = np.where(np.arange(lo, hi)[None, :] > qpos[:, None], -np.inf, S)
        m_new = np.maximum(m, S.max(axis=1))
        ref = np.where(np.isfinite(m_new), m_new, 0.0)   # safe exponent reference
        alpha = np.exp(m - ref)                 # rescale of the old state
        p = np.exp(S - ref[:, None])
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ v[lo:hi]
        m = m_new
        if trace is not None:
            trace.append((m.copy(), l.copy()))

    out = np.zeros_like(o)
    live = l > 0
    out[live] = o[live] / l[live][:, None]
    lse = np.full(nq, -np.inf)
    lse[live] = m[live] + np.log(l[live])
    return out, lse
