"""CPU tests that pin the backward oracle (``oracle/attention_bwd_ref.py``).

No GPU needed.  The definition and the tiled method pass every pin of
``oracle_bwd_pins``; planted mistakes in a copy of the definition each fail at
least one pin.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle_bwd_pins as pins
from oracle import (all_compositions, attention_bwd_dq_rows_ref, attention_bwd_kv_rows_ref,
                    attention_bwd_ref,
                    attention_bwd_ref_batched,
                    attention_bwd_tiled_ref, uniform_bounds)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_definition_passes_pin(pin):
    with np.errstate(all="raise"):
        pin(attention_bwd_ref)


@pytest.mark.parametrize("qt,kt", [(1, 1), (2, 3), (4, 64), (64, 1)])
def test_tiled_method_passes_every_pin(qt, kt):
    def impl(q, k, v, do, scale, causal, off):
        return attention_bwd_tiled_ref(q, k, v, do, scale, uniform_bounds(len(q), qt),
                                       uniform_bounds(len(k), kt), causal, off)
    assert pins.run_pins(impl) == []


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_definition_under_every_key_tiling(causal):
    rng = np.random.default_rng(31 + causal)
    for nk in range(1, 7):
        nq = nk + 1
        q, k = rng.standard_normal((nq, 3)) * 2, rng.standard_normal((nk, 3)) * 2
        v, g = rng.standard_normal((nk, 2)), rng.standard_normal((nq, 2))
        ref = attention_bwd_ref(q, k, v, g, 0.8, causal, 1)
        for kb in all_compositions(nk):
            for qb in ([0, nq], uniform_bounds(nq, 2)):
                got = attention_bwd_tiled_ref(q, k, v, g, 0.8, qb, kb, causal, 1)
                for a, b in zip(got, ref):
                    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_batched_rows_match_per_head():
    rng = np.random.default_rng(40)
    B, H, N, d = 2, 3, 37, 8
    q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    qr = np.array([0, 5, 36, 17])
    kr = np.array([36, 0, 1, 20])
    for causal in (False, True):
        dq, dk, dv = attention_bwd_ref_batched(q, k, v, g, 0.4, causal, qr, kr,
                                               heads=[4, 1], chunk=8)
        for n, flat in enumerate([4, 1]):
            b, h = divmod(flat, H)
            rq, rk, rv = attention_bwd_ref(q[b, h], k[b, h], v[b, h], g[b, h], 0.4, causal)
            np.testing.assert_allclose(dq[n], rq[qr], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dk[n], rk[kr], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv[n], rv[kr], rtol=0, atol=1e-12)


# A copy of the definition with switches that plant one mistake each.
def _generic(q, k, v, do, scale, causal, off, *, correction="p_weighted", sign=1.0,
             scale_dq=True, scale_dk=True, transpose_dv=True, transpose_dk=True,
             dq_from="k", dv_from="p", mask="future"):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = scale * (q @ k.T)
    i = np.arange(len(q))[:, None] + off
    j = np.arange(len(k))[None, :]
    if causal:
        s = np.where((j > i) if mask == "future" else (j >= i), -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = do @ v.T
    r = {"p_weighted": (dp * p).sum(axis=1, keepdims=True),
         "unweighted": dp.sum(axis=1, keepdims=True),
         "none": 0.0}[correction]
    ds = p * (dp - sign * r)
    dv = (p.T @ do) if transpose_dv else (p @ do)
    if dv_from == "ds":
        dv = ds.T @ do
    dk = (ds.T @ q) if transpose_dk else (ds @ q)
    dq = ds @ (k if dq_from == "k" else v)
    return (scale * dq if scale_dq else dq), (scale * dk if scale_dk else dk), dv


MUTANTS = {
    "no_correction": dict(correction="none"),
    "unweighted_correction": dict(correction="unweighted"),
    "correction_sign": dict(sign=-1.0),
    "dq_unscaled": dict(scale_dq=False),
    "dk_unscaled": dict(scale_dk=False),
    "dv_not_transposed": dict(transpose_dv=False),
    "dk_not_transposed": dict(transpose_dk=False),
    "dq_from_values": dict(dq_from="v"),
    "dv_from_ds": dict(dv_from="ds"),
    "mask_off_by_one": dict(mask="off_by_one"),
}


@pytest.mark.parametrize("causal,offset,nq,nk", [(False, 0, 40, 40), (True, 0, 40, 40),
                                                 (True, 25, 15, 40), (False, 0, 9, 30)])
def test_dq_rows_equal_the_definition(causal, offset, nq, nk):
    """attention_bwd_dq_rows_ref on chosen rows against attention_bwd_ref's full dQ."""
    rng = np.random.default_rng(41)
    q = rng.standard_normal((nq, 6))
    k = rng.standard_normal((nk, 6))
    v = rng.standard_normal((nk, 5))
    g = rng.standard_normal((nq, 5))
    rows = np.array([0, 3, nq - 1])
    full = attention_bwd_ref(q, k, v, g, 0.45, causal, offset)[0]
    got = attention_bwd_dq_rows_ref(q, k, v, g, 0.45, causal, rows, offset)
    np.testing.assert_allclose(got, full[rows], rtol=0, atol=1e-13)


def test_kv_rows_of_causal_tail_equal_the_definition():
    """Causal: keys j >= j0 are seen only by queries i >= j0, so summing over
    those queries gives the full dK and dV rows; other query sets do not."""
    rng = np.random.default_rng(43)
    n = 60
    q, k, v, g = (rng.standard_normal((n, 6)) for _ in range(4))
    dq, dk, dv = attention_bwd_ref(q, k, v, g, 0.5, True)
    keys = np.arange(48, n)
    got_k, got_v = attention_bwd_kv_rows_ref(q, k, v, g, 0.5, True, keys, np.arange(48, n))
    np.testing.assert_allclose(got_k, dk[keys], rtol=0, atol=1e-13)
    np.testing.assert_allclose(got_v, dv[keys], rtol=0, atol=1e-13)
    short_k, _ = attention_bwd_kv_rows_ref(q, k, v, g, 0.5, True, keys, np.arange(50, n))
    assert np.abs(short_k - dk[keys]).max() > 1e-3


def test_generic_copy_is_sound():
    assert pins.run_pins(lambda *a: _generic(*a)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    failed = pins.run_pins(lambda *a: _generic(*a, **MUTANTS[name]))
    assert failed, "mutant %s passed every pin" % name
