"""CPU tests that pin the oracle to what the pages and mathematics fix.

No GPU needed.  The oracle (``oracle/``) is checked against fixed values and
properties (``oracle_pins``), and planted mistakes in copies of it are shown to
be caught by at least one pin.
"""
from __future__ import annotations

import json
import math

import numpy as np
import pytest
import torch

import oracle_pins as pins
from oracle import (all_compositions, attention_ref, attention_ref_batched, bf16_bits_to_f64,
                    f32_scale, online_attention_ref, uniform_bounds)


def _two_pass(q, k, v, scale, causal):
    return attention_ref(q, k, v, scale, causal)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    with np.errstate(all="raise"):
        pin(_two_pass)


@pytest.mark.parametrize("tile", [1, 2, 3, 64])
def test_online_recurrence_passes_every_pin(tile):
    def impl(q, k, v, scale, causal):
        return online_attention_ref(q, k, v, scale, uniform_bounds(len(k), tile), causal)
    assert pins.run_pins(impl) == []


def test_worked_example_running_state():
    """State after each tile equals the page's numbers (sec. 22.7)."""
    g = json.load(open(pins.GOLDEN))
    s = [t[0] for t in g["scores_per_tile"]]
    q = np.array([[1.0]])
    k = np.array([[s[0]], [s[1]]])
    v = np.array([[1.0], [0.0]])
    trace = []
    o, lse = online_attention_ref(q, k, v, 1.0, [0, 1, 2], trace=trace)
    st = g["state_after_tile"]
    assert trace[0][0][0] == st[0]["m"] and trace[0][1][0] == st[0]["l"]
    l2 = sum(math.exp(t["exp_of"]) if "exp_of" in t else t["const"] for t in st[1]["l_terms"])
    assert trace[1][0][0] == st[1]["m"]
    assert abs(trace[1][1][0] - l2) < 1e-15
    # v = (1, 0): the output is the first key's final weight, i.e. its rescale / l
    assert abs(o[0, 0] - math.exp(g["rescale_of_first_contribution"]["exp_of"]) / l2) < 1e-15


def test_worked_example_needs_the_max():
    """Without subtracting a running max the first exponential already overflows."""
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float64(1000.0)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("offset", [0, 2])
def test_recurrence_equals_two_pass_under_every_tiling(causal, offset):
    """Brute force: all 2**(Nk-1) ways to cut the keys, tiny shapes."""
    rng = np.random.default_rng(100 + offset + causal)
    for nk in range(1, 8):
        nq = max(1, nk - 1)
        q = rng.standard_normal((nq, 3)) * 3
        k = rng.standard_normal((nk, 3)) * 3
        v = rng.standard_normal((nk, 2))
        ro, rl = attention_ref(q, k, v, 0.7, causal, query_offset=offset)
        count = 0
        for bounds in all_compositions(nk):
            o, lse = online_attention_ref(q, k, v, 0.7, bounds, causal, query_offset=offset)
            np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)
            count += 1
        assert count == 2 ** (nk - 1)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_tile_sweep(causal):
    """Tile widths 1, 4 and wider than the key axis agree (sec. 22.7 experiment)."""
    rng = np.random.default_rng(7)
    nk = 11
    q = rng.standard_normal((nk, 5))
    k = rng.standard_normal((nk, 5))
    v = rng.standard_normal((nk, 3))
    ro, rl = attention_ref(q, k, v, 1 / math.sqrt(5), causal)
    for tile in (1, 2, 4, nk, nk + 1):
        o, lse = online_attention_ref(q, k, v, 1 / math.sqrt(5), uniform_bounds(nk, tile), causal)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_fully_hidden_rows_policy():
    """Rows that see no key: output 0 and LSE -inf, no NaN (lab policy, sec. 22.7)."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((5, 3))
    k = rng.standard_normal((5, 3))
    v = rng.standard_normal((5, 2))
    with np.errstate(invalid="raise"):
        o, lse = attention_ref(q, k, v, 1.0, True, query_offset=-2)
        oo, ol = online_attention_ref(q, k, v, 1.0, [0, 2, 5], True, query_offset=-2)
    assert np.all(o[:2] == 0) and np.all(np.isneginf(lse[:2]))
    assert np.all(oo[:2] == 0) and np.all(np.isneginf(ol[:2]))
    np.testing.assert_allclose(oo, o, atol=1e-12)
    np.testing.assert_allclose(ol[2:], lse[2:], atol=1e-12)
    # row 2 (absolute position 0) sees exactly key 0
    np.testing.assert_allclose(o[2], v[0], atol=1e-12)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((40, 8))
    k = rng.standard_normal((40, 8))
    v = rng.standard_normal((40, 8))
    rows = np.array([0, 3, 17, 39])
    for causal in (False, True):
        o, lse = attention_ref(q, k, v, 0.3, causal)
        os_, ls = attention_ref(q, k, v, 0.3, causal, rows=rows)
        np.testing.assert_array_equal(os_, o[rows])
        np.testing.assert_array_equal(ls, lse[rows])


def test_batched_matches_per_head():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((2, 3, 10, 4))
    k = rng.standard_normal((2, 3, 10, 4))
    v = rng.standard_normal((2, 3, 10, 4))
    o, lse = attention_ref_batched(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            oh, lh = attention_ref(q[b, h], k[b, h], v[b, h], 0.5, True)
            np.testing.assert_array_equal(o[b, h], oh)
            np.testing.assert_array_equal(lse[b, h], lh)


def test_bf16_decoding_matches_torch_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = bf16_bits_to_f64(bits)
    theirs = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], theirs[~nan])
    assert bf16_bits_to_f64(np.array([0x3F80], dtype=np.uint16))[0] == 1.0
    assert bf16_bits_to_f64(np.array([0xC000], dtype=np.uint16))[0] == -2.0


def test_f32_scale():
    assert f32_scale(0.125) == 0.125
    s = f32_scale(1 / math.sqrt(128))
    assert s == float(np.float32(1 / math.sqrt(128))) and s != 1 / math.sqrt(128)


# ---------------------------------------------------------------------------
# Planted mistakes: each broken copy of the definition must fail some pin.
# ---------------------------------------------------------------------------

def _generic(q, k, v, scale, causal, *, use_scale=True, subtract_max=True, lse_mode="ln",
             mask="future", normalise=True, value_rows=None, axis=1):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s = (scale if use_scale else 1.0) * (q @ k.T)
    i = np.arange(len(q))[:, None]
    j = np.arange(len(k))[None, :]
    if causal:
        hide = {"future": j > i, "past": j < i, "off_by_one": j >= i}[mask]
        s = np.where(hide, -np.inf, s)
    m = s.max(axis=1, keepdims=True) if subtract_max else np.zeros((len(q), 1))
    p = np.exp(s - m)
    l = p.sum(axis=axis, keepdims=True)
    vv = v if value_rows is None else v[value_rows(len(v))]
    o = p @ vv
    if normalise:
        o = o / l if axis == 1 else (p / l) @ vv
    lse = {"ln": m[:, 0] + np.log(l.ravel()[:len(q)]) if axis == 1 else m[:, 0],
           "no_max": np.log(l[:, 0]) if axis == 1 else m[:, 0],
           "log2": m[:, 0] + np.log2(l.ravel()[:len(q)])}[lse_mode]
    return o, lse


MUTANTS = {
    "drop_scale": dict(use_scale=False),
    "no_max_subtraction": dict(subtract_max=False),
    "lse_without_max": dict(lse_mode="no_max"),
    "lse_log2": dict(lse_mode="log2"),
    "mask_reversed": dict(mask="past"),
    "mask_off_by_one": dict(mask="off_by_one"),
    "no_normalise": dict(normalise=False),
    "values_reversed": dict(value_rows=lambda n: np.arange(n)[::-1]),
    "normalise_wrong_axis": dict(axis=0),
}


def test_generic_copy_is_sound():
    """The mutant generator with no mutation passes every pin (so failures below
    are caused by the planted mistake alone)."""
    assert pins.run_pins(lambda *a: _generic(*a)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    kw = MUTANTS[name]
    failed = pins.run_pins(lambda *a: _generic(*a, **kw))
    assert failed, "mutant %s passed every pin" % name


def _online_mutant(q, k, v, scale, causal, bounds, *, rescale_o=True, rescale_l=True,
                   safe=True, query_offset=0):
    """The per-row recurrence with one step optionally broken: the old o or l
    not rescaled by exp(m - m'), or no safe reference for still-hidden rows."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    out = np.zeros((len(q), v.shape[1]))
    lse = np.zeros(len(q))
    for i in range(len(q)):
        m, l, o = -math.inf, 0.0, np.zeros(v.shape[1])
        for first, end in zip(bounds[:-1], bounds[1:]):
            s = [(-math.inf if causal and j > i + query_offset else scale * float(q[i] @ k[j]))
                 for j in range(first, end)]
            m_next = max(m, max(s))
            ref = m_next if (m_next != -math.inf or not safe) else 0.0
            keep = math.exp(m - ref) if not (math.isinf(m) and math.isinf(ref)) else math.nan
            w = np.exp(np.array(s) - ref)
            l = (keep if rescale_l else 1.0) * l + w.sum()
            o = (keep if rescale_o else 1.0) * o + w @ v[first:end]
            m = m_next
        out[i] = o / l
        lse[i] = m + math.log(l) if l > 0 else -math.inf
    return out, lse


@pytest.mark.parametrize("kw", [dict(rescale_o=False), dict(rescale_l=False)],
                         ids=["no_alpha_on_o", "no_alpha_on_l"])
def test_recurrence_without_rescale_is_caught(kw):
    failed = pins.run_pins(
        lambda q, k, v, s, c: _online_mutant(q, k, v, s, c, uniform_bounds(len(k), 1), **kw))
    assert "pin_worked_example" in failed


def test_recurrence_without_safe_max_gives_nan_on_hidden_rows():
    q = np.ones((3, 1))
    k = np.ones((3, 1))
    v = np.ones((3, 1))
    with np.errstate(all="ignore"):
        o, _ = _online_mutant(q, k, v, 1.0, True, [0, 1, 3], safe=False, query_offset=-1)
        oo, _ = online_attention_ref(q, k, v, 1.0, [0, 1, 3], True, query_offset=-1)
    assert np.isnan(o[0]).any()
    assert not np.isnan(oo).any()


# ---- general shapes: query offset, Nq != Nk, dv != d (sec. 22.7 lab conventions) ----

GENERAL_CASES = [  # (nq, nk, d, dv, offset, causal)
    (1, 9, 4, 3, 8, True),      # one decoding step at the last position
    (3, 11, 5, 2, 4, True),     # a chunk of queries in the middle
    (7, 4, 3, 6, 0, True),      # more queries than keys: later rows see every key
    (6, 6, 4, 4, 2, True),
    (5, 8, 2, 7, 0, False),
]


@pytest.mark.parametrize("case", GENERAL_CASES)
def test_general_shapes_match_torch(case):
    """Offset causal mask, Nq != Nk and dv != d against torch's float64 SDPA
    with an explicit boolean mask (key j visible iff j <= i + offset)."""
    import torch.nn.functional as F
    nq, nk, d, dv, off, causal = case
    rng = np.random.default_rng(60 + nq + nk)
    q, k, v = (rng.standard_normal(s) for s in ((nq, d), (nk, d), (nk, dv)))
    mask = torch.from_numpy(np.arange(nk)[None, :] <= np.arange(nq)[:, None] + off) if causal else None
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None], attn_mask=mask, scale=0.45)[0]
    o, lse = attention_ref(q, k, v, 0.45, causal, query_offset=off)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    s = 0.45 * q @ k.T
    if causal:
        s = np.where(mask.numpy(), s, -np.inf)
    np.testing.assert_allclose(lse, np.log(np.exp(s).sum(axis=1)), rtol=0, atol=1e-12)


def test_query_chunk_equals_rows_of_full_problem():
    """Queries at positions off .. off+nq-1 against nk = off + nq keys give the
    last nq rows of the square causal problem (decoding-style subproblem)."""
    rng = np.random.default_rng(70)
    n, nq = 13, 4
    q, k, v = (rng.standard_normal((n, 3)) for _ in range(3))
    full_o, full_l = attention_ref(q, k, v, 0.8, True)
    o, lse = attention_ref(q[n - nq:], k, v, 0.8, True, query_offset=n - nq)
    np.testing.assert_allclose(o, full_o[n - nq:], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, full_l[n - nq:], rtol=0, atol=1e-14)


def test_offset_past_last_key_is_unmasked():
    rng = np.random.default_rng(71)
    q, k, v = rng.standard_normal((4, 3)), rng.standard_normal((6, 3)), rng.standard_normal((6, 2))
    a = attention_ref(q, k, v, 0.7, True, query_offset=5)
    b = attention_ref(q, k, v, 0.7, False)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-15)


def test_no_keys_policy():
    o, lse = attention_ref(np.ones((3, 4)), np.zeros((0, 4)), np.zeros((0, 2)), 0.5, True,
                           query_offset=1)
    assert o.shape == (3, 2) and np.all(o == 0) and np.all(np.isneginf(lse))
