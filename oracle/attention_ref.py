"""Plain two-pass softmax attention in float64 -- the parity oracle.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct CPU
definition that the GPU path is checked against.  Only the test-suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never does, and this module imports nothing from the product
(no kernels, headers, helpers or constants are shared).

What it computes (page "22. GPU Engineering: Correctness, Throughput, and
Attention", sec. 22.5 and the worked lab of sec. 22.7; page "GPU Programming &
Kernel Development", Classic kernels: the two-pass softmax):

    S      = scale * Q K^T                      (scores of every query row)
    S[i,j] = -inf  where key j is in the future  (causal; mask before max/sum)
    m_i    = max_j S[i,j]                        (pass 1)
    P      = exp(S - m),  l_i = sum_j P[i,j]     (pass 2)
    O      = (P V) / l,   LSE_i = m_i + ln(l_i)  (natural log of the
                                                  normaliser of the *scaled*
                                                  scores)

The online (tiled) method of sec. 22.5 reaches exactly this result in real
arithmetic; the oracle is therefore the plain definition, not the recurrence.

Causal rule (sec. 22.7 lab, the score masking step): with absolute query
positions ``i + query_offset``, key ``j`` is hidden when ``j > i +
query_offset``.  A row whose keys are all hidden follows the lab's stated
policy: output row 0 and LSE -inf.

Inputs are the same bf16-quantised values the GPU receives, widened exactly to
float64 (sec. 22.3 asks for a reference on the same quantised inputs); the
scale is the float32 value the GPU receives, widened to float64.
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_bits_to_f64", "f32_scale", "attention_ref", "attention_ref_batched"]


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode raw bfloat16 bit patterns (uint16) to float64, exactly.

    A bfloat16 is the upper half of an IEEE-754 binary32: sign, 8 exponent
    bits, 7 stored mantissa bits.  Shifting the 16 bits into the top of a
    32-bit word and reinterpreting it as binary32 gives the value exactly;
    widening binary32 to binary64 is exact as well.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("expected uint16 bit patterns, got %s" % b.dtype)
    with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_scale(scale: float) -> float:
    """The float32 value a caller's scale becomes at the C boundary, as float64."""
    return float(np.float64(np.float32(scale)))


def _visible(nq: int, nk: int, causal: bool, query_offset: int, rows) -> np.ndarray:
    """Boolean [len(rows), nk]: True where key j may be attended by query row i.

    sec. 22.7 lab: a key is hidden when its position exceeds the query's
    absolute position (query index plus the offset).
    """
    rows = np.asarray(rows)
    if not causal:
        return np.ones((rows.size, nk), dtype=bool)
    key_pos = np.arange(nk)[None, :]
    query_pos = (rows + query_offset)[:, None]
    return key_pos <= query_pos


def attention_ref(q, k, v, scale: float, causal: bool = False, rows=None,
                  query_offset: int = 0):
    """Two-pass float64 attention for ONE head.

    q: [Nq, d], k: [Nk, d], v: [Nk, dv] -- float arrays (widened to float64).
    scale: multiplies Q K^T (used as given; pass ``f32_scale(s)`` to mirror a
           float32 boundary).
    rows: optional 1-D integer array of query rows to evaluate (default: all).
    Returns (O [len(rows), dv] float64, LSE [len(rows)] float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 2 or k.ndim != 2 or v.ndim != 2:
        raise ValueError("q, k, v must be rank 2 for one head")
    if q.shape[1] != k.shape[1] or k.shape[0] != v.shape[0]:
        raise ValueError("incompatible q/k/v shapes")
    nq, nk = q.shape[0], k.shape[0]
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    if rows.ndim != 1 or (rows.size and (rows.min() < 0 or rows.max() >= nq)):
        raise ValueError("rows out of range")

    # Scores of the selected rows; a library matmul is one step of the definition.
    s = float(scale) * (q[rows] @ k.T)
    vis = _visible(nq, nk, causal, query_offset, rows)
    s = np.where(vis, s, -np.inf)

    # Pass 1: row maximum over visible keys.
    m = s.max(axis=1) if nk else np.full(rows.size, -np.inf)
    live = np.isfinite(m)                       # rows with at least one visible key
    m_ref = np.where(live, m, 0.0)              # any finite reference for dead rows

    # Pass 2: exponentials, normaliser, weighted values.
    p = np.exp(s - m_ref[:, None])              # exp(-inf) = 0 on hidden keys
    l = p.sum(axis=1)
    o = np.zeros((rows.size, v.shape[1]), dtype=np.float64)
    o[live] = (p[live] @ v) / l[live][:, None]
    lse = np.full(rows.size, -np.inf)
    lse[live] = m[live] + np.log(l[live])
    return o, lse


def attention_ref_batched(q, k, v, scale: float, causal: bool = False, rows=None):
    """attention_ref over every (batch, head) of [B, H, N, d] arrays.

    rows: None (all rows), a 1-D array used for every head, or a
    [B*H, R] integer array giving the rows of each head in (b, h) order.
    Returns (O [B, H, R, d], LSE [B, H, R]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if q.ndim != 4:
        raise ValueError("expected [B, H, N, d]")
    B, H, N, _ = q.shape
    if rows is None:
        per_head = [np.arange(N)] * (B * H)
    else:
        r = np.asarray(rows, dtype=np.int64)
        per_head = [r] * (B * H) if r.ndim == 1 else [r[i] for i in range(B * H)]
    R = per_head[0].size
    o = np.empty((B, H, R, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            i = b * H + h
            o[b, h], lse[b, h] = attention_ref(q[b, h], k[b, h], v[b, h], scale, causal,
                                               rows=per_head[i])
    return o, lse
