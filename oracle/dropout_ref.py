"""Attention with dropout on the probabilities -- oracle side.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU leg
may use it; nothing is shared with the HIP path).

Page "22. GPU Engineering: Correctness, Throughput, and Attention", sec. 22.5:
dropout is to be added only after the masks are defined reproducibly.  The
definition used here (this library's reading; the pages give none):

* Generator: Philox-4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011): a 128-bit counter (four
  32-bit words) and a 64-bit key (two words); each round multiplies words 0
  and 2 by fixed odd constants into 64-bit products and mixes their halves
  with words 1 and 3 and the key; the key is advanced by two Weyl constants
  between rounds.  (32-bit words: one block is 16 random bytes for about 80
  32-bit vector operations on the GPU; the 64-bit variant needs emulated
  128-bit products.)
* Mask: for head n = b*H + h, the query at absolute position i and key j,
      word = Philox(counter = (i, j >> 4, n, 0), key = (seed mod 2^32, seed >> 32))
      byte = bits 8 (j mod 4) .. +7 of word[(j >> 2) mod 4]   (byte j mod 16, little endian)
      keep(i, j) = byte >= t,    drop probability t / 256,  t in 0..255.
* Output: O = (P * M) V / (1 - t/256) with P the softmax of the scaled, masked
  scores (the normaliser counts every visible key, kept or dropped); LSE is the
  undropped log-normaliser.  t = 0 keeps everything and is plain attention.
* General shapes (the lab's decoding-style subproblems of sec. 22.7): query row
  r of a chunk that starts at position ``query_offset`` is the query at
  absolute position query_offset + r, both for the causal rule and for the
  mask counter, so a chunk's outputs are the corresponding rows of the whole
  problem with the same seed.
* Gradients (the chain rule through the mask): with Pd = P * M / (1 - t/256),
  dV = Pd^T G, dP = (G V^T) * M / (1 - t/256), dS = P * (dP - rowsum(dP * P)),
  dQ = scale dS K, dK = scale dS^T Q; rowsum(dP * P) still equals
  rowsum(G * O) (the sec. 22.7 identity applied to O = Pd V).
"""
from __future__ import annotations

import numpy as np

from .attention_ref import _visible

__all__ = ["philox4x32", "dropout_keep", "attention_dropout_ref", "attention_dropout_bwd_ref",
           "attention_dropout_bwd_ref_rows"]

_M0 = 0xD2511F53
_M1 = 0xCD9E8D57
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def philox4x32(counter, key, rounds: int = 10):
    """Philox-4x32 block for one counter (4 ints) and key (2 ints): 4 ints."""
    x0, x1, x2, x3 = (int(c) & _MASK32 for c in counter)
    k0, k1 = (int(k) & _MASK32 for k in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + _W0) & _MASK32
            k1 = (k1 + _W1) & _MASK32
        p0 = _M0 * x0
        p1 = _M1 * x2
        hi0, lo0 = p0 >> 32, p0 & _MASK32
        hi1, lo1 = p1 >> 32, p1 & _MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def _philox4x32_arrays(x0, x1, x2, x3, k0: int, k1: int, rounds: int = 10):
    """philox4x32 over broadcast numpy counter words (uint64 arrays holding
    32-bit values, so each 32 x 32-bit product is exact)."""
    x0, x1, x2, x3 = (np.asarray(x, dtype=np.uint64) & np.uint64(_MASK32) for x in (x0, x1, x2, x3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    for r in range(rounds):
        if r:
            k0 = (k0 + _W0) & _MASK32
            k1 = (k1 + _W1) & _MASK32
        p0 = np.uint64(_M0) * x0
        p1 = np.uint64(_M1) * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK32)
        x0, x1, x2, x3 = hi1 ^ x1 ^ np.uint64(k0), lo1, hi0 ^ x3 ^ np.uint64(k1), lo0
    return x0, x1, x2, x3


def dropout_keep(n_head: int, rows, nk: int, seed: int, t: int) -> np.ndarray:
    """Boolean keep mask [len(rows), nk] of head n_head (flat b*H + h): the
    blocks for counters (row, block, n_head, 0), block = 0 .. ceil(nk/16) - 1,
    evaluated as arrays, each block's four words read as 16 little-endian bytes."""
    rows = np.asarray(rows, dtype=np.int64)
    if t == 0 or rows.size == 0 or nk == 0:
        return np.ones((rows.size, nk), dtype=bool)
    nb = (nk + 15) // 16
    words = _philox4x32_arrays(rows[:, None], np.arange(nb)[None, :], n_head, 0,
                               seed & _MASK32, (seed >> 32) & _MASK32)
    block = np.stack(words, axis=-1).astype("<u4")                  # [R, nb, 4]
    raw = block.view(np.uint8).reshape(rows.size, nb * 16)[:, :nk]  # byte j of the row
    return raw >= t


def _probs(q, k, scale, causal, rows, query_offset=0):
    """(P[rows], LSE[rows]); a row that sees no key (no keys at all) gets P = 0
    and LSE = -inf (the lab's policy)."""
    s = float(scale) * (q[rows] @ k.T)
    s = np.where(_visible(q.shape[0], k.shape[0], causal, query_offset, rows), s, -np.inf)
    m = s.max(axis=1) if k.shape[0] else np.full(len(rows), -np.inf)
    live = np.isfinite(m)
    p = np.exp(s - np.where(live, m, 0.0)[:, None])
    l = p.sum(axis=1)
    p[live] /= l[live][:, None]
    p[~live] = 0.0
    lse = np.full(len(rows), -np.inf)
    lse[live] = m[live] + np.log(l[live])
    return p, lse


def attention_dropout_ref(q, k, v, scale: float, causal: bool, n_head: int, seed: int, t: int,
                          rows=None, query_offset: int = 0):
    """One head: (O [R, dv], LSE [R]) with the dropout mask above, float64.
    q [Nq, d], k [Nk, d], v [Nk, dv]; query r sits at position query_offset + r."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    p, lse = _probs(q, k, scale, causal, rows, query_offset)
    keep = dropout_keep(n_head, rows + query_offset, k.shape[0], seed, t)
    return (p * keep) @ v / (1.0 - t / 256.0), lse


def attention_dropout_bwd_ref(q, k, v, do, scale: float, causal: bool, n_head: int, seed: int,
                              t: int, query_offset: int = 0):
    """One head: (dQ, dK, dV) of sum(G * O) with O from attention_dropout_ref
    (same shapes and offset)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    rows = np.arange(q.shape[0])
    p, _ = _probs(q, k, scale, causal, rows, query_offset)
    mk = dropout_keep(n_head, rows + query_offset, k.shape[0], seed, t) / (1.0 - t / 256.0)
    dv = (p * mk).T @ do
    dp = (do @ v.T) * mk
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    return float(scale) * (ds @ k), float(scale) * (ds.T @ q), dv


def attention_dropout_bwd_ref_rows(q, k, v, do, scale: float, causal: bool, n_head: int,
                                   seed: int, t: int, query_rows=None, key_rows=None,
                                   chunk: int = 1024, query_offset: int = 0):
    """One head: attention_dropout_bwd_ref's dQ[query_rows], dK[key_rows] and
    dV[key_rows] (None: all rows), the same formulas evaluated for a chunk of
    query rows at a time so long sequences fit in memory."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    n = q.shape[0]
    qr = np.arange(n) if query_rows is None else np.asarray(query_rows, dtype=np.int64)
    kr = np.arange(k.shape[0]) if key_rows is None else np.asarray(key_rows, dtype=np.int64)
    dq = np.zeros((qr.size, q.shape[1]))
    dk = np.zeros((kr.size, k.shape[1]))
    dv = np.zeros((kr.size, v.shape[1]))
    for c0 in range(0, n, chunk):
        rows = np.arange(c0, min(n, c0 + chunk))
        p, _ = _probs(q, k, scale, causal, rows, query_offset)
        mk = dropout_keep(n_head, rows + query_offset, k.shape[0], seed, t) / (1.0 - t / 256.0)
        dp = (do[rows] @ v.T) * mk
        ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
        dv += (p * mk)[:, kr].T @ do[rows]
        dk += float(scale) * (ds[:, kr].T @ q[rows])
        sel = (qr >= c0) & (qr <= rows[-1])
        if sel.any():
            dq[sel] = float(scale) * (ds[qr[sel] - c0] @ k)
    return dq, dk, dv
