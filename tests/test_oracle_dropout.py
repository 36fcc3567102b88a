"""CPU pins of the dropout oracle: the Philox-4x64-10 generator against numpy's
independent implementation, the mask statistics, t = 0 reducing to plain
attention, and the gradients through the mask against finite differences and
torch float64 autograd."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import (attention_bwd_ref, attention_dropout_bwd_ref, attention_dropout_ref,
                    attention_ref, dropout_keep, philox4x64)


def _numpy_philox(counter, key):
    """numpy's Philox-4x64-10: the state counter is advanced (256-bit, with
    carry) before each block, so start one below the wanted counter."""
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=words, key=np.array(key, dtype=np.uint64))
    return tuple(int(x) for x in bg.random_raw(4))


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 2, 3, 4), (5, 7)),
    ((8191, 255, 63, 0), (123456789, 0)),
    ((0, 1, 0, 0), (2 ** 64 - 1, 2 ** 63)),          # numpy's start needs a borrow
    ((2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1), (3, 4)),
])
def test_philox_matches_numpy(counter, key):
    assert philox4x64(counter, key) == _numpy_philox(counter, key)


def test_philox_random_counters_match_numpy():
    rng = np.random.default_rng(7)
    for _ in range(50):
        c = tuple(int(x) for x in rng.integers(0, 2 ** 63, 4))
        k = tuple(int(x) for x in rng.integers(0, 2 ** 63, 2))
        assert philox4x64(c, k) == _numpy_philox(c, k)


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
