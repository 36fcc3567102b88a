"""Gradients of softmax attention in float64 -- the backward parity oracle.

TEST INFRASTRUCTURE ONLY (same rules as ``attention_ref``: tests, the smoke
check and the benchmark's CPU leg may use it; the product never does; nothing
is shared with the HIP path).

What it computes (page "22. GPU Engineering: Correctness, Throughput, and
Attention", sec. 22.5 last paragraph and sec. 22.7 derivation).  For one head
with P = softmax(S), S = scale Q K^T (future keys hidden when causal), O = P V
and an upstream gradient G = dL/dO:

    dV = P^T G                 dP = G V^T
    dS = P * (dP - r)          r_i = sum_j dP[i,j] P[i,j]   (a softmax row's
                                                              Jacobian is
                                                              diag(p) - p p^T)
    dQ = scale dS K            dK = scale dS^T Q

Functions:

* ``attention_bwd_ref`` -- that definition for one head: the full probability
  matrix from the two-pass softmax, and r from dP and P directly.
* ``attention_bwd_tiled_ref`` -- the memory-saving method of sec. 22.7: r
  taken through the output (the page shows sum_j dP[i,j] P[i,j] =
  sum_c G[i,c] O[i,c]) and each probability block recomputed as exp(S - LSE)
  from the saved per-row log-normaliser, organised as two passes (key tiles
  accumulate dK and dV, then query tiles accumulate dQ).  It is pinned against
  the definition under many tilings.
* ``attention_bwd_ref_batched`` -- the definition over [B, H, N, d] arrays,
  evaluating dQ only on chosen query rows and dK, dV only on chosen key rows
  (query rows are taken in chunks to bound memory; that only splits the sums
  over queries into partial sums).

Rows that see no key follow the lab's policy: zero probabilities, hence zero
gradient contributions.  Inputs are the same bf16-quantised values the GPU
receives, widened exactly to float64.
"""
from __future__ import annotations

import numpy as np

from .attention_ref import _visible, attention_ref

__all__ = ["attention_bwd_ref", "attention_bwd_tiled_ref", "attention_bwd_ref_batched",
           "attention_bwd_dq_rows_ref", "attention_bwd_kv_rows_ref"]


def _as64(*xs):
    return tuple(np.asarray(x, dtype=np.float64) for x in xs)


def _softmax_rows(q, k, scale, causal, query_offset, rows):
    """P[rows, :] by the two-pass definition; rows with no visible key -> 0."""
    s = float(scale) * (q[rows] @ k.T)
    s = np.where(_visible(q.shape[0], k.shape[0], causal, query_offset, rows), s, -np.inf)
    m = s.max(axis=1) if k.shape[0] else np.full(len(rows), -np.inf)
    live = np.isfinite(m)
    p = np.exp(s - np.where(live, m, 0.0)[:, None])
    p[~live] = 0.0
    p[live] /= p[live].sum(axis=1, keepdims=True)
    return p


def _check(q, k, v, do):
    if q.ndim != 2 or k.ndim != 2 or v.ndim != 2 or do.ndim != 2:
        raise ValueError("q, k, v, dO must be rank 2 for one head")
    if q.shape[1] != k.shape[1] or k.shape[0] != v.shape[0]:
        raise ValueError("incompatible q/k/v shapes")
    if do.shape != (q.shape[0], v.shape[1]):
        raise ValueError("dO must be [Nq, dv]")


def attention_bwd_ref(q, k, v, do, scale: float, causal: bool = False, query_offset: int = 0):
    """(dQ, dK, dV) of a loss L with dL/dO = ``do``, one head, float64.

    q: [Nq, d], k: [Nk, d], v: [Nk, dv], do: [Nq, dv].
    """
    q, k, v, do = _as64(q, k, v, do)
    _check(q, k, v, do)
    p = _softmax_rows(q, k, scale, causal, query_offset, np.arange(q.shape[0]))
    dv = p.T @ do
    dp = do @ v.T
    r = (dp * p).sum(axis=1, keepdims=True)
    ds = p * (dp - r)
    return float(scale) * (ds @ k), float(scale) * (ds.T @ q), dv


def attention_bwd_tiled_ref(q, k, v, do, scale: float, q_bounds, k_bounds,
                            causal: bool = False, query_offset: int = 0):
    """The recomputing backward of sec. 22.7, organised in two passes over a grid
    of query tiles [q_bounds[a], q_bounds[a+1]) and key tiles [k_bounds[b],
    k_bounds[b+1]).  It keeps only the forward's per-row log-normaliser and
    output, never the probability matrix:

    * per row, the correction r_i = sum_c G[i,c] O[i,c] (the page's identity
      for sum_j dP[i,j] P[i,j]);
    * pass 1, one key tile at a time: its dK and dV rows are summed over every
      query tile, each probability block rebuilt as exp(S - LSE);
    * pass 2, one query tile at a time: its dQ rows are summed over every key
      tile, rebuilding the same blocks.
    At most one probability block exists at a time."""
    q, k, v, do = _as64(q, k, v, do)
    _check(q, k, v, do)
    out, lse = attention_ref(q, k, v, scale, causal, query_offset=query_offset)
    r = (do * out).sum(axis=1)
    q_tiles = list(zip(q_bounds[:-1], q_bounds[1:]))
    k_tiles = list(zip(k_bounds[:-1], k_bounds[1:]))

    def block(qa, qb, ka, kb):
        """(P, dS) of query rows qa..qb-1 against keys ka..kb-1."""
        s = float(scale) * (q[qa:qb] @ k[ka:kb].T)
        if causal:
            hidden = np.arange(ka, kb)[None, :] > (np.arange(qa, qb) + query_offset)[:, None]
            s = np.where(hidden, -np.inf, s)
        rows_lse = lse[qa:qb]
        seen = np.isfinite(rows_lse)              # rows with no visible key: P = 0
        prob = np.zeros_like(s)
        prob[seen] = np.exp(s[seen] - rows_lse[seen][:, None])
        dprob = do[qa:qb] @ v[ka:kb].T
        return prob, prob * (dprob - r[qa:qb, None])

    dk, dv = np.zeros_like(k), np.zeros_like(v)
    for ka, kb in k_tiles:                        # pass 1: key tiles own dK, dV
        for qa, qb in q_tiles:
            prob, dscore = block(qa, qb, ka, kb)
            dv[ka:kb] += prob.T @ do[qa:qb]
            dk[ka:kb] += float(scale) * (dscore.T @ q[qa:qb])
    dq = np.zeros_like(q)
    for qa, qb in q_tiles:                        # pass 2: query tiles own dQ
        for ka, kb in k_tiles:
            _, dscore = block(qa, qb, ka, kb)
            dq[qa:qb] += float(scale) * (dscore @ k[ka:kb])
    return dq, dk, dv


def attention_bwd_ref_batched(q, k, v, do, scale: float, causal: bool = False,
                              query_rows=None, key_rows=None, heads=None, chunk: int = 1024):
    """The definition over [B, H, N, d] inputs (self-attention, query_offset 0).

    query_rows / key_rows: None (all rows) or 1-D integer arrays used for every
    evaluated head.  heads: None (all B*H heads) or a list of flat head indices
    b*H + h.  Returns (dQ [nh, Rq, d], dK [nh, Rk, d], dV [nh, Rk, dv]) for the
    evaluated heads in the given order.
    """
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    if q.ndim != 4:
        raise ValueError("expected [B, H, N, d]")
    B, H, N, _ = q.shape
    heads = list(range(B * H)) if heads is None else list(heads)
    qr = np.arange(N) if query_rows is None else np.asarray(query_rows, dtype=np.int64)
    kr = np.arange(N) if key_rows is None else np.asarray(key_rows, dtype=np.int64)
    dv_dim = v.shape[-1]
    dq = np.zeros((len(heads), qr.size, q.shape[-1]))
    dk = np.zeros((len(heads), kr.size, k.shape[-1]))
    dvo = np.zeros((len(heads), kr.size, dv_dim))
    for n, flat in enumerate(heads):
        b, h = divmod(flat, H)
        qh, kh, vh, gh = _as64(q[b, h], k[b, h], v[b, h], do[b, h])
        _check(qh, kh, vh, gh)
        for c0 in range(0, N, chunk):
            rows = np.arange(c0, min(N, c0 + chunk))
            p = _softmax_rows(qh, kh, scale, causal, 0, rows)
            dp = gh[rows] @ vh.T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dvo[n] += p[:, kr].T @ gh[rows]
            dk[n] += float(scale) * (ds[:, kr].T @ qh[rows])
            sel = (qr >= c0) & (qr < rows[-1] + 1)
            if sel.any():
                dq[n, sel] = float(scale) * (ds[qr[sel] - c0] @ kh)
    return dq, dk, dvo


def attention_bwd_dq_rows_ref(q, k, v, do, scale: float, causal: bool = False, rows=None,
                              query_offset: int = 0):
    """dQ[rows] of attention_bwd_ref for one head.  Row i of dQ depends only on
    row i of P, dP and dS, so the definition restricted to the chosen rows
    needs no other query: P_i by the two-pass softmax, dP_i = G_i V^T,
    dS_i = P_i * (dP_i - sum_j dP_ij P_ij), dQ_i = scale dS_i K."""
    q, k, v, do = _as64(q, k, v, do)
    _check(q, k, v, do)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    p = _softmax_rows(q, k, scale, causal, query_offset, rows)
    dp = do[rows] @ v.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    return float(scale) * (ds @ k)


def attention_bwd_kv_rows_ref(q, k, v, do, scale: float, causal: bool, key_rows, query_rows,
                              query_offset: int = 0):
    """dK[key_rows], dV[key_rows] of attention_bwd_ref for one head, summing the
    key columns of dS and P over `query_rows` only:
        dV_j = sum_i P_ij G_i,   dK_j = scale sum_i dS_ij q_i   (i in query_rows).
    Exact when query_rows holds every query that sees the keys (under the
    causal mask with offset 0, keys j >= j0 are seen only by queries i >= j0)."""
    q, k, v, do = _as64(q, k, v, do)
    _check(q, k, v, do)
    kr = np.asarray(key_rows, dtype=np.int64)
    qr = np.asarray(query_rows, dtype=np.int64)
    p = _softmax_rows(q, k, scale, causal, query_offset, qr)
    dp = do[qr] @ v.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    return float(scale) * (ds[:, kr].T @ q[qr]), p[:, kr].T @ do[qr]
