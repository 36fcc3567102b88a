"""Pins for a one-head attention backward, independent of its own code.

Each pin takes ``impl(q, k, v, do, scale, causal, query_offset) -> (dQ, dK, dV)``
(float64 numpy, one head) and raises when the implementation disagrees with
something fixed from outside it: derivatives of the forward definition taken
numerically, an independent autograd library, closed forms, and invariants of
softmax attention.  ``run_pins`` returns the names of the failed pins, so the
tests can show that the oracle passes all of them and that planted mistakes
fail at least one.

Source of the method: page "22. GPU Engineering: Correctness, Throughput, and
Attention", sec. 22.5 (backward formulas) and sec. 22.7 (derivation, finite
difference experiment).
"""
from __future__ import annotations

import numpy as np

from oracle import attention_ref


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise AssertionError("%s: shape %s vs %s" % (what, a.shape, b.shape))
    err = np.max(np.abs(a - b), initial=0.0)
    if not err <= tol:
        raise AssertionError("%s: max error %.3e > %.1e" % (what, err, tol))


def _loss(q, k, v, g, scale, causal, off):
    o, _ = attention_ref(q, k, v, scale, causal, query_offset=off)
    return float((g * o).sum())


# (nq, nk, d, dv, scale, causal, query_offset, input spread)
FD_CASES = [
    (4, 4, 3, 3, 0.7, False, 0, 1.0),
    (6, 6, 4, 4, 0.5, True, 0, 1.0),
    (3, 7, 4, 2, 0.45, True, 4, 1.0),    # decode-style: 3 queries at positions 4..6
    (5, 9, 2, 5, -0.6, False, 0, 1.0),   # negative scale, dv != d
    (5, 5, 3, 3, 1.0, True, 0, 4.0),     # large logits: sharp softmax
]


def _case_inputs(seed, nq, nk, d, dv, spread):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((nq, d)) * spread, rng.standard_normal((nk, d)) * spread,
            rng.standard_normal((nk, dv)), rng.standard_normal((nq, dv)), rng)


def pin_finite_differences(impl):
    """Directional derivatives of sum(G * O), O from the forward definition, by
    central differences (the experiment sec. 22.7 prescribes), for Q, K and V
    separately, in several random directions each."""
    h = 1e-5
    for n, (nq, nk, d, dv, scale, causal, off, spread) in enumerate(FD_CASES):
        q, k, v, g, rng = _case_inputs(300 + n, nq, nk, d, dv, spread)
        grads = impl(q, k, v, g, scale, causal, off)
        for which, x in enumerate((q, k, v)):
            for _ in range(3):
                e = rng.standard_normal(x.shape)
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which] = x + h * e
                args_m[which] = x - h * e
                fd = (_loss(*args_p, g, scale, causal, off)
                      - _loss(*args_m, g, scale, causal, off)) / (2 * h)
                an = float((grads[which] * e).sum())
                tol = 1e-7 * (1.0 + np.abs(grads[which]).sum() * np.abs(e).max())
                if not abs(fd - an) <= tol:
                    raise AssertionError("finite difference d%s case %d: %.10g vs %.10g"
                                         % ("QKV"[which], n, fd, an))


def pin_torch_autograd(impl):
    """torch float64 autograd through its scaled-dot-product attention."""
    import torch
    import torch.nn.functional as F
    for n, (nq, nk, d, dv, scale, causal, off, spread) in enumerate(FD_CASES):
        q, k, v, g, _ = _case_inputs(400 + n, nq, nk, d, dv, spread)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        mask = None
        if causal:
            mask = torch.from_numpy(np.arange(nk)[None, :] <= np.arange(nq)[:, None] + off)
        out = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=mask,
                                             scale=scale)[0]
        out.backward(torch.from_numpy(g))
        dq, dk, dv_ = impl(q, k, v, g, scale, causal, off)
        _close(dq, tq.grad.numpy(), 1e-12, "autograd dQ")
        _close(dk, tk.grad.numpy(), 1e-12, "autograd dK")
        _close(dv_, tv.grad.numpy(), 1e-12, "autograd dV")


def pin_two_keys_closed_form(impl):
    """One query, two keys, d = dv = 1: P = (s, 1 - s) with s the logistic of
    scale*q*(a - b); differentiate O = s x + (1 - s) y by hand."""
    for (qv, a, b, x, y, gv, scale) in ((1.3, 0.4, -0.9, 2.0, -1.0, 0.7, 0.8),
                                        (-0.5, 2.0, 1.5, 0.25, 3.0, -1.2, 1.7)):
        s = 1.0 / (1.0 + np.exp(-scale * qv * (a - b)))
        ds = s * (1 - s)                     # derivative of the logistic
        dq_ = gv * ds * scale * (a - b) * (x - y)
        dka = gv * ds * scale * qv * (x - y)
        dq, dk, dv = impl(np.array([[qv]]), np.array([[a], [b]]), np.array([[x], [y]]),
                          np.array([[gv]]), scale, False, 0)
        _close(dq, [[dq_]], 1e-13, "two keys dQ")
        _close(dk, [[dka], [-dka]], 1e-13, "two keys dK")
        _close(dv, [[gv * s], [gv * (1 - s)]], 1e-13, "two keys dV")


def pin_one_key(impl):
    """A single key gets probability one whatever the scores: dQ = dK = 0 and
    dV is the sum of the output gradients."""
    rng = np.random.default_rng(21)
    q, k = rng.standard_normal((5, 4)), rng.standard_normal((1, 4))
    v, g = rng.standard_normal((1, 3)), rng.standard_normal((5, 3))
    for causal in (False, True):
        dq, dk, dv = impl(q, k, v, g, 0.9, causal, 0)
        _close(dq, np.zeros_like(q), 1e-14, "one key dQ")
        _close(dk, np.zeros_like(k), 1e-14, "one key dK")
        _close(dv, g.sum(axis=0, keepdims=True), 1e-13, "one key dV")


def pin_zero_scale(impl):
    """scale = 0: uniform weights over the visible keys, so dQ = dK = 0 and
    dV[j] = sum over the queries i that see j of G[i] / (number of keys i sees)."""
    rng = np.random.default_rng(22)
    q, k = rng.standard_normal((6, 3)), rng.standard_normal((6, 3))
    v, g = rng.standard_normal((6, 2)), rng.standard_normal((6, 2))
    for causal in (False, True):
        dq, dk, dv = impl(q, k, v, g, 0.0, causal, 0)
        w = np.array([[1.0 / (i + 1) if j <= i else 0.0 for j in range(6)] for i in range(6)]) \
            if causal else np.full((6, 6), 1.0 / 6)
        _close(dq, np.zeros_like(q), 1e-14, "zero scale dQ")
        _close(dk, np.zeros_like(k), 1e-14, "zero scale dK")
        _close(dv, w.T @ g, 1e-13, "zero scale dV")


def pin_invariants(impl):
    """Softmax ignores a common shift of a row's scores, so adding one vector to
    every key changes nothing: the dK rows sum to zero.  Adding one vector to
    every value adds it to every output: the dV rows sum to the sum of G.
    Scores are bilinear in Q and K: sum dQ*Q = sum dK*K."""
    for n, (nq, nk, d, dv, scale, causal, off, spread) in enumerate(FD_CASES):
        q, k, v, g, _ = _case_inputs(500 + n, nq, nk, d, dv, spread)
        dq, dk, dv_ = impl(q, k, v, g, scale, causal, off)
        _close(dk.sum(axis=0), np.zeros(d), 1e-12, "key shift")
        _close(dv_.sum(axis=0), g.sum(axis=0), 1e-12, "value shift")
        _close((dq * q).sum(), (dk * k).sum(), 1e-12, "scale symmetry")


def pin_mp_brute_force(impl):
    """Every gradient entry of tiny cases by central differences of a 50-digit
    evaluation of the forward definition (step 1e-20, error far below 1e-13)."""
    import mpmath
    mpmath.mp.dps = 50

    def loss(q, k, v, g, scale, causal):
        tot = mpmath.mpf(0)
        for i in range(len(q)):
            keys = [j for j in range(len(k)) if not (causal and j > i)]
            e = {j: mpmath.e ** (scale * mpmath.fsum(a * b for a, b in zip(q[i], k[j])))
                 for j in keys}
            z = mpmath.fsum(e.values())
            for c in range(len(v[0])):
                tot += g[i][c] * mpmath.fsum(e[j] * v[j][c] for j in keys) / z
        return tot

    rng = np.random.default_rng(23)
    h = mpmath.mpf("1e-20")
    for (n, d, dv, scale, causal) in ((2, 2, 1, 0.9, False), (3, 2, 2, -0.7, True)):
        q, k, v, g = (rng.standard_normal(s) * 1.5 for s in ((n, d), (n, d), (n, dv), (n, dv)))
        mp = [[[mpmath.mpf(float(x)) for x in row] for row in a] for a in (q, k, v, g)]
        sc = mpmath.mpf(scale)
        grads = impl(q, k, v, g, scale, causal, 0)
        for which in range(3):
            ref = np.zeros(grads[which].shape)
            for i in range(ref.shape[0]):
                for c in range(ref.shape[1]):
                    plus = [[list(r) for r in a] for a in mp[:3]]
                    minus = [[list(r) for r in a] for a in mp[:3]]
                    plus[which][i][c] += h
                    minus[which][i][c] -= h
                    ref[i, c] = float((loss(*plus, mp[3], sc, causal)
                                       - loss(*minus, mp[3], sc, causal)) / (2 * h))
            _close(grads[which], ref, 1e-13, "50-digit d%s" % "QKV"[which])


ALL_PINS = [pin_finite_differences, pin_torch_autograd, pin_two_keys_closed_form, pin_one_key,
            pin_zero_scale, pin_invariants, pin_mp_brute_force]


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
