"""CPU pins of the dropout oracle: the Philox-4x32-10 generator against the
published known-answer vectors, the byte order of the mask, the mask
statistics, t = 0 reducing to plain attention, and the gradients through the
mask against finite differences and torch float64 autograd."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from oracle import (attention_bwd_ref, attention_dropout_bwd_ref, attention_dropout_bwd_ref_rows,
                    attention_dropout_ref, attention_ref, dropout_keep, philox4x32)

_KAT = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")))


def _hex(words):
    return tuple(int(w, 16) for w in words)


@pytest.mark.parametrize("i", range(len(_KAT["vectors"])))
def test_philox_known_answers(i):
    v = _KAT["vectors"][i]
    assert philox4x32(_hex(v["counter"]), _hex(v["key"])) == _hex(v["out"])


def test_philox_known_answers_reject_other_round_counts():
    v = _KAT["vectors"][2]
    for rounds in (7, 9, 11):
        assert philox4x32(_hex(v["counter"]), _hex(v["key"]), rounds) != _hex(v["out"])


def test_mask_bytes_are_the_little_endian_block():
    """keep[i, j] is byte j mod 16 of the block (row i, j // 16, head, 0) laid
    out as four little-endian 32-bit words; the seed's low word is key word 0."""
    seed, head, t = (7 << 32) | 12345, 5, 100
    rows, nk = np.array([0, 3, 70000]), 45
    keep = dropout_keep(head, rows, nk, seed, t)
    for a, i in enumerate(rows):
        for blk in range(3):
            raw = np.array(philox4x32((int(i), blk, head, 0), (12345, 7)), dtype="<u4").tobytes()
            for jj in range(16):
                j = 16 * blk + jj
                if j < nk:
                    assert keep[a, j] == (raw[jj] >= t)


def test_mask_matches_scalar_generator_on_random_positions():
    """The array evaluation of dropout_keep against one scalar block per element."""
    rng = np.random.default_rng(21)
    for _ in range(3):
        seed = int(rng.integers(0, 2 ** 63)) * 2 + 1
        head, t = int(rng.integers(0, 2 ** 31)), int(rng.integers(1, 256))
        rows = rng.integers(0, 2 ** 31, 5)
        nk = int(rng.integers(1, 300))
        keep = dropout_keep(head, rows, nk, seed, t)
        for a, i in enumerate(rows):
            for j in rng.integers(0, nk, 20):
                w = philox4x32((int(i), int(j) >> 4, head, 0), (seed & 0xFFFFFFFF, seed >> 32))
                byte = (w[(int(j) >> 2) & 3] >> (8 * (int(j) & 3))) & 0xFF
                assert keep[a, j] == (byte >= t)


@pytest.mark.parametrize("t", [1, 64, 128, 230])
def test_keep_fraction(t):
    keep = dropout_keep(3, np.arange(200), 500, seed=11, t=t)
    n, p = keep.size, 1 - t / 256
    assert abs(keep.mean() - p) <= 5 * np.sqrt(p * (1 - p) / n)


def test_masks_depend_on_seed_head_and_position():
    a = dropout_keep(0, np.arange(64), 96, 1, 128)
    assert not np.array_equal(a, dropout_keep(0, np.arange(64), 96, 2, 128))
    assert not np.array_equal(a, dropout_keep(1, np.arange(64), 96, 1, 128))
    assert np.array_equal(a[10:20], dropout_keep(0, np.arange(10, 20), 96, 1, 128))


def test_zero_threshold_is_plain_attention():
    rng = np.random.default_rng(8)
    q, k, v, g = (rng.standard_normal((9, 4)) for _ in range(4))
    for causal in (False, True):
        o, l = attention_dropout_ref(q, k, v, 0.6, causal, 2, 99, 0)
        ro, rl = attention_ref(q, k, v, 0.6, causal)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l, rl, rtol=0, atol=1e-14)
        for a, b in zip(attention_dropout_bwd_ref(q, k, v, g, 0.6, causal, 2, 99, 0),
                        attention_bwd_ref(q, k, v, g, 0.6, causal)):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_dropout_gradients_match_finite_differences():
    rng = np.random.default_rng(9)
    q, k, v, g = (rng.standard_normal((7, 5)) for _ in range(4))
    grads = attention_dropout_bwd_ref(q, k, v, g, 0.5, True, 4, 31, 100)
    h = 1e-5
    for which in range(3):
        for _ in range(3):
            e = rng.standard_normal((7, 5))
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[which] = [q, k, v][which] + h * e
            args_m[which] = [q, k, v][which] - h * e
            fp = (g * attention_dropout_ref(*args_p, 0.5, True, 4, 31, 100)[0]).sum()
            fm = (g * attention_dropout_ref(*args_m, 0.5, True, 4, 31, 100)[0]).sum()
            assert abs((fp - fm) / (2 * h) - (grads[which] * e).sum()) < 1e-7


def test_dropout_gradients_match_torch_autograd():
    rng = np.random.default_rng(10)
    n, d = 33, 6
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    t = 77
    keep = torch.from_numpy(dropout_keep(1, np.arange(n), n, 5, t).astype(np.float64))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = 0.4 * tq @ tk.T
    s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    o = (torch.softmax(s, dim=1) * keep / (1 - t / 256)) @ tv
    o.backward(torch.from_numpy(g))
    ref_o, _ = attention_dropout_ref(q, k, v, 0.4, True, 1, 5, t)
    np.testing.assert_allclose(ref_o, o.detach().numpy(), rtol=0, atol=1e-12)
    for a, b in zip(attention_dropout_bwd_ref(q, k, v, g, 0.4, True, 1, 5, t),
                    (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=0, atol=1e-12)


def test_correction_identity_holds_under_dropout():
    """rowsum(dP * P) equals rowsum(G * O) with the dropped output O."""
    rng = np.random.default_rng(12)
    q, k, v, g = (rng.standard_normal((20, 4)) for _ in range(4))
    t = 90
    o, _ = attention_dropout_ref(q, k, v, 0.7, True, 0, 3, t)
    s = 0.7 * q @ k.T
    s = np.where(np.tri(20, dtype=bool), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    mk = dropout_keep(0, np.arange(20), 20, 3, t) / (1 - t / 256)
    dp = (g @ v.T) * mk
    np.testing.assert_allclose((dp * p).sum(axis=1), (g * o).sum(axis=1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_chunked_rows_equal_the_definition(causal):
    """attention_dropout_bwd_ref_rows (chunks of query rows, sampled outputs)
    against attention_dropout_bwd_ref on the same inputs."""
    rng = np.random.default_rng(13)
    n, d = 50, 6
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    full = attention_dropout_bwd_ref(q, k, v, g, 0.3, causal, 6, 17, 70)
    qr, kr = np.array([0, 7, 16, 49]), np.array([1, 15, 33, 48])
    part = attention_dropout_bwd_ref_rows(q, k, v, g, 0.3, causal, 6, 17, 70, qr, kr, chunk=16)
    for a, b in zip(part, (full[0][qr], full[1][kr], full[2][kr])):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# ---- expectation over seeds: the keep scale and the all-keys normaliser ----
#
# Each probability is kept with probability pi = (256 - t) / 256 (a byte >= t
# of a uniform byte), so E[keep_j] = pi and, with the normaliser counting every
# visible key, E[O] = sum_j P_j v_j * keep_scale * pi, which is the plain
# attention output exactly when keep_scale = 256 / (256 - t).  Over S seeds the
# seed-mean of O then lies within a CLT bound of plain attention: the per-seed
# variance of one element is keep_scale^2 pi (1 - pi) sum_j P_j^2 v_j^2 (the
# mask bytes of different keys are independent draws of the generator).  Two
# other readings -- no keep scale, or a normaliser over the kept keys only --
# miss the same bound.

_SEEDS = 4000


def _expectation_case(t, causal):
    rng = np.random.default_rng(40 + t)
    q, k, v = (rng.standard_normal((5, 3)) for _ in range(3))
    o, lse = attention_ref(q, k, v, 0.8, causal)
    p = np.exp(0.8 * q @ k.T - lse[:, None])
    if causal:
        p = np.tril(p)
    pi = (256 - t) / 256.0
    ks = 256.0 / (256 - t)
    sigma = np.sqrt(ks * ks * pi * (1 - pi) * (p * p) @ (v * v))      # per-seed std of O
    return q, k, v, o, lse, p, sigma


def _seed_mean(fn, n_seeds=_SEEDS):
    return sum(fn(seed) for seed in range(1000, 1000 + n_seeds)) / n_seeds


@pytest.mark.parametrize("t", [64, 128, 192])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_output_is_unbiased_over_seeds(t, causal):
    q, k, v, o, lse, p, sigma = _expectation_case(t, causal)
    lses = []

    def one(seed):
        od, ld = attention_dropout_ref(q, k, v, 0.8, causal, 3, seed, t)
        lses.append(ld)
        return od

    mean = _seed_mean(one)
    bound = 5.0 * sigma / np.sqrt(_SEEDS) + 1e-12
    assert np.all(np.abs(mean - o) <= bound), np.max(np.abs(mean - o) / bound)
    # The log-normaliser counts every visible key: the same for every mask.
    assert all(np.array_equal(ld, lse) for ld in lses)


@pytest.mark.parametrize("t", [64, 128, 192])
def test_other_dropout_readings_miss_the_expectation(t):
    """Planted readings on the oracle's own masks: no 1/(1 - t/256) factor, or
    the normaliser taken over kept keys only (a ratio whose mean is not the
    plain output); each misses the bound the oracle meets."""
    q, k, v, o, lse, p, sigma = _expectation_case(t, False)
    bound = 5.0 * sigma / np.sqrt(_SEEDS) + 1e-12
    pi = (256 - t) / 256.0

    def unscaled(seed):
        od, _ = attention_dropout_ref(q, k, v, 0.8, False, 3, seed, t)
        return od * pi                          # the same masks without the keep scale

    def kept_keys_only(seed):
        keep = dropout_keep(3, np.arange(5), 5, seed, t)
        w = p * keep
        den = w.sum(axis=1, keepdims=True)
        return np.where(den > 0, w @ v / np.where(den > 0, den, 1.0), 0.0)

    for fn in (unscaled, kept_keys_only):
        assert np.any(np.abs(_seed_mean(fn) - o) > bound), fn.__name__


# ---- general shapes (query offset, Nq != Nk, dv != d) ---------------------------
#
# Query r of a chunk starting at position `query_offset` is the query at
# absolute position query_offset + r, for the causal rule and for the mask
# counter alike, so a chunk is the corresponding rows of the whole problem.

GENERAL_DROP = [  # (nq, nk, d, dv, offset, causal)
    (1, 40, 4, 3, 39, True),     # one decoding step at the last position
    (5, 37, 5, 2, 20, True),     # a chunk in the middle
    (9, 6, 3, 6, 0, True),       # more queries than keys
    (6, 33, 4, 4, 0, False),     # cross attention, no mask
]


@pytest.mark.parametrize("nq,nk,d,dv,off,causal", GENERAL_DROP)
def test_general_zero_threshold_is_plain_attention(nq, nk, d, dv, off, causal):
    rng = np.random.default_rng(nq + nk)
    q, k = rng.standard_normal((nq, d)), rng.standard_normal((nk, d))
    v, g = rng.standard_normal((nk, dv)), rng.standard_normal((nq, dv))
    o, l = attention_dropout_ref(q, k, v, 0.6, causal, 2, 99, 0, query_offset=off)
    ro, rl = attention_ref(q, k, v, 0.6, causal, query_offset=off)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-14)
    for a, b in zip(attention_dropout_bwd_ref(q, k, v, g, 0.6, causal, 2, 99, 0, query_offset=off),
                    attention_bwd_ref(q, k, v, g, 0.6, causal, query_offset=off)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("t", [26, 128])
def test_query_chunk_is_rows_of_the_whole_problem(t):
    """A chunk of queries at positions 11..17 over all 30 keys (causal) gives the
    outputs, LSE and dQ rows of the square problem's rows 11..17."""
    rng = np.random.default_rng(60 + t)
    q, k, v, g = (rng.standard_normal((30, 4)) for _ in range(4))
    o, l = attention_dropout_ref(q, k, v, 0.7, True, 5, 1234, t)
    oc, lc = attention_dropout_ref(q[11:18], k, v, 0.7, True, 5, 1234, t, query_offset=11)
    np.testing.assert_allclose(oc, o[11:18], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lc, l[11:18], rtol=0, atol=1e-14)
    dq = attention_dropout_bwd_ref(q, k, v, g, 0.7, True, 5, 1234, t)[0]
    dqc = attention_dropout_bwd_ref(q[11:18], k, v, g[11:18], 0.7, True, 5, 1234, t,
                                    query_offset=11)[0]
    np.testing.assert_allclose(dqc, dq[11:18], rtol=0, atol=1e-13)


@pytest.mark.parametrize("nq,nk,d,dv,off,causal", GENERAL_DROP)
def test_general_gradients_match_finite_differences(nq, nk, d, dv, off, causal):
    rng = np.random.default_rng(70 + nq)
    q, k = rng.standard_normal((nq, d)), rng.standard_normal((nk, d))
    v, g = rng.standard_normal((nk, dv)), rng.standard_normal((nq, dv))
    args = [q, k, v]
    grads = attention_dropout_bwd_ref(q, k, v, g, 0.5, causal, 4, 31, 100, query_offset=off)
    h = 1e-5
    for which in range(3):
        e = rng.standard_normal(args[which].shape)
        ap, am = list(args), list(args)
        ap[which] = args[which] + h * e
        am[which] = args[which] - h * e
        fp = (g * attention_dropout_ref(*ap, 0.5, causal, 4, 31, 100, query_offset=off)[0]).sum()
        fm = (g * attention_dropout_ref(*am, 0.5, causal, 4, 31, 100, query_offset=off)[0]).sum()
        assert abs((fp - fm) / (2 * h) - (grads[which] * e).sum()) < 1e-7


def test_no_keys_gives_the_lab_policy():
    q = np.ones((3, 4))
    o, l = attention_dropout_ref(q, np.zeros((0, 4)), np.zeros((0, 2)), 0.5, False, 0, 1, 26)
    assert np.array_equal(o, np.zeros((3, 2))) and np.all(l == -np.inf)
