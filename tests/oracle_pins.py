"""Pins for a one-head attention implementation, independent of its own code.

Each pin takes ``impl(q, k, v, scale, causal) -> (O, LSE)`` (float64 numpy,
one head) and raises AssertionError when the implementation disagrees with
something the pages or plain mathematics fix.  ``run_pins`` returns the names
of the pins that failed, so tests can show both that the oracle passes every
pin and that a planted mistake (a dropped term, a wrong sign or index, a
transposed operand) fails at least one.

Sources: page "22. GPU Engineering: Correctness, Throughput, and Attention"
(sec. 22.5 recurrence and masking rule; sec. 22.7 worked example and lab
conventions) and page "GPU Programming & Kernel Development" (Classic kernels:
softmax).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_22_7.json")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise AssertionError("%s: shape %s vs %s" % (what, a.shape, b.shape))
    if not np.all(np.isfinite(a) == np.isfinite(b)):
        raise AssertionError("%s: finiteness differs" % what)
    fin = np.isfinite(b)
    if not np.array_equal(a[~fin], b[~fin]):
        raise AssertionError("%s: non-finite values differ" % what)
    err = np.max(np.abs(a[fin] - b[fin]), initial=0.0)
    if not err <= tol:
        raise AssertionError("%s: max error %.3e > %.1e" % (what, err, tol))


def _golden_value(spec) -> float:
    if "exp_of" in spec:
        return math.exp(spec["exp_of"])
    return float(spec["const"])


def pin_worked_example(impl):
    """Two scores 1000 and 1001 (sec. 22.7): weights exp(-1) and 1 over 1+exp(-1)."""
    g = json.load(open(GOLDEN))
    s = [t[0] for t in g["scores_per_tile"]]
    l_final = sum(_golden_value(t) for t in g["state_after_tile"][1]["l_terms"])
    m_final = g["state_after_tile"][1]["m"]
    rescale = _golden_value(g["rescale_of_first_contribution"])
    q = np.array([[1.0]])
    k = np.array([[s[0]], [s[1]]])
    v = np.array([[2.0, -1.0, 0.5], [-3.0, 4.0, 0.25]])
    o, lse = impl(q, k, v, 1.0, False)
    _close(o[0], (rescale * v[0] + v[1]) / l_final, 1e-12, "worked example O")
    _close(lse, [m_final + math.log(l_final)], 1e-9, "worked example LSE")


def pin_one_key(impl):
    """A single visible key: O is that key's value row, LSE its scaled score."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 4))
    k = rng.standard_normal((1, 4))
    v = rng.standard_normal((1, 5))
    for causal in (False, True):
        o, lse = impl(q, k, v, 0.7, causal)
        _close(o, np.repeat(v, 3, axis=0), 1e-12, "one key O")
        _close(lse, 0.7 * (q @ k[0]), 1e-12, "one key LSE")


def pin_zero_scale(impl):
    """scale 0: uniform weights over visible keys -> (prefix) mean, LSE = ln(count)."""
    rng = np.random.default_rng(12)
    n = 9
    q = rng.standard_normal((n, 3))
    k = rng.standard_normal((n, 3))
    v = rng.standard_normal((n, 4))
    o, lse = impl(q, k, v, 0.0, False)
    _close(o, np.repeat(v.mean(axis=0, keepdims=True), n, axis=0), 1e-12, "zero scale O")
    _close(lse, np.full(n, math.log(n)), 1e-12, "zero scale LSE")
    o, lse = impl(q, k, v, 0.0, True)
    counts = np.arange(1, n + 1)
    _close(o, np.cumsum(v, axis=0) / counts[:, None], 1e-12, "zero scale causal O")
    _close(lse, np.log(counts), 1e-12, "zero scale causal LSE")


def pin_causal_first_row(impl):
    """Causal row 0 sees only key 0 (sec. 22.7 masking rule)."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((6, 5))
    k = rng.standard_normal((6, 5))
    v = rng.standard_normal((6, 3))
    o, lse = impl(q, k, v, 0.9, True)
    _close(o[0], v[0], 1e-12, "causal row 0 O")
    _close(lse[0], 0.9 * q[0] @ k[0], 1e-12, "causal row 0 LSE")
    # the last row sees every key: equals the non-causal result for that row
    o2, lse2 = impl(q, k, v, 0.9, False)
    _close(o[-1], o2[-1], 1e-12, "causal last row O")
    _close(lse[-1], lse2[-1], 1e-12, "causal last row LSE")


def pin_rows_sum_to_one(impl):
    """V = identity makes O the probability matrix: rows are >= 0 and sum to 1."""
    rng = np.random.default_rng(14)
    n = 7
    q = rng.standard_normal((5, 3)) * 3
    k = rng.standard_normal((n, 3)) * 3
    for causal in (False, True):
        p, _ = impl(q, k, np.eye(n), 0.5, causal)
        if p.min() < 0:
            raise AssertionError("negative probability")
        _close(p.sum(axis=1), np.ones(5), 1e-12, "row sums")
        if causal:
            hidden = np.arange(n)[None, :] > np.arange(5)[:, None]
            if np.any(p[hidden] != 0):
                raise AssertionError("hidden key has weight")


def pin_constant_v(impl):
    """Every value row equal to c gives O = c on every row."""
    rng = np.random.default_rng(15)
    q = rng.standard_normal((6, 4)) * 5
    k = rng.standard_normal((8, 4)) * 5
    c = rng.standard_normal(3)
    for causal in (False, True):
        o, _ = impl(q, k, np.tile(c, (8, 1)), 1.3, causal)
        _close(o, np.tile(c, (6, 1)), 1e-12, "constant V")


def pin_score_shift(impl):
    """Adding c to every score of a row leaves O and adds c to LSE.

    Realised by appending one dimension: q gets c/scale, every key gets 1.
    """
    rng = np.random.default_rng(16)
    q = rng.standard_normal((5, 3))
    k = rng.standard_normal((7, 3))
    v = rng.standard_normal((7, 2))
    scale, c = 0.8, np.array([0.0, 2.5, -4.0, 10.0, 0.3])
    for causal in (False, True):
        o1, l1 = impl(q, k, v, scale, causal)
        q2 = np.concatenate([q, (c / scale)[:, None]], axis=1)
        k2 = np.concatenate([k, np.ones((7, 1))], axis=1)
        o2, l2 = impl(q2, k2, v, scale, causal)
        _close(o2, o1, 1e-12, "shift O")
        _close(l2, l1 + c, 1e-12, "shift LSE")


def pin_permutations(impl):
    """Non-causal: permuting K and V rows together changes nothing; permuting Q
    rows permutes O and LSE the same way."""
    rng = np.random.default_rng(17)
    q = rng.standard_normal((6, 4))
    k = rng.standard_normal((9, 4))
    v = rng.standard_normal((9, 3))
    o, lse = impl(q, k, v, 0.6, False)
    pk = rng.permutation(9)
    o2, lse2 = impl(q, k[pk], v[pk], 0.6, False)
    _close(o2, o, 1e-12, "key permutation O")
    _close(lse2, lse, 1e-12, "key permutation LSE")
    pq = rng.permutation(6)
    o3, lse3 = impl(q[pq], k, v, 0.6, False)
    _close(o3, o[pq], 1e-12, "query permutation O")
    _close(lse3, lse[pq], 1e-12, "query permutation LSE")


def pin_torch_sdpa(impl):
    """torch's float64 CPU scaled-dot-product attention, an independent routine."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(18)
    for (nq, nk, d, dv) in ((5, 5, 4, 4), (13, 13, 8, 3), (33, 33, 16, 16)):
        q = rng.standard_normal((nq, d))
        k = rng.standard_normal((nk, d))
        v = rng.standard_normal((nk, dv))
        for causal in (False, True):
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
                is_causal=causal, scale=0.37)[0].numpy()
            o, _ = impl(q, k, v, 0.37, causal)
            _close(o, ref, 1e-12, "torch sdpa O")


def _brute(q, k, v, scale, causal):
    """50-digit brute force with plain loops (mpmath), one visible set per row."""
    import mpmath
    mpmath.mp.dps = 50
    nq, nk, dv = len(q), len(k), len(v[0])
    O, L = [], []
    for i in range(nq):
        keys = [j for j in range(nk) if not (causal and j > i)]
        s = {j: mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b)
                                                  for a, b in zip(q[i], k[j])) for j in keys}
        e = {j: mpmath.e ** s[j] for j in keys}
        z = mpmath.fsum(e.values())
        O.append([float(mpmath.fsum(e[j] * mpmath.mpf(v[j][c]) for j in keys) / z)
                  for c in range(dv)])
        L.append(float(mpmath.log(z)))
    return np.array(O), np.array(L)


def pin_brute_force(impl):
    """Tiny random cases against a 50-digit evaluation of the softmax definition."""
    rng = np.random.default_rng(19)
    for (n, d, dv, scale) in ((1, 1, 1, 1.0), (3, 2, 2, 0.5), (5, 3, 2, 1.7), (6, 2, 3, -0.8)):
        q = rng.standard_normal((n, d)) * 2
        k = rng.standard_normal((n, d)) * 2
        v = rng.standard_normal((n, dv))
        for causal in (False, True):
            ro, rl = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)
            o, lse = impl(q, k, v, scale, causal)
            _close(o, ro, 1e-12, "brute force O")
            _close(lse, rl, 1e-12, "brute force LSE")


ALL_PINS = [pin_worked_example, pin_one_key, pin_zero_scale, pin_causal_first_row,
            pin_rows_sum_to_one, pin_constant_v, pin_score_shift, pin_permutations,
            pin_torch_sdpa, pin_brute_force]


def run_pins(impl):
    """Names of the pins ``impl`` fails (an exception of any kind is a failure)."""
    failed = []
    with np.errstate(all="ignore"):
        for pin in ALL_PINS:
            try:
                pin(impl)
            except Exception:  # noqa: BLE001 - any error means the pin rejects impl
                failed.append(pin.__name__)
    return failed
