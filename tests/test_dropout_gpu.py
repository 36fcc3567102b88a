"""GPU parity of attention with dropout (attn_fwd_dropout, attn_bwd_dropout)
against the float64 oracle, which draws the same Philox-4x32-10 mask on the
CPU.

Bars.  drop_t = 0 keeps every probability: the output must equal attn_fwd's
bit for bit.  Otherwise O = keep_scale * (a masked form of the plain sum) with
keep_scale = 256 / (256 - drop_t), so its absolute error is keep_scale times
that of the plain forward:
    max |dO| <= 1e-2 keep_scale,  mean |dO| <= 1e-3 keep_scale,
    max |dLSE| <= 1e-3            (LSE counts every visible key: unchanged).
A wrong mask byte moves an output by the full weight of one key times
keep_scale, far above these bars.

The backward runs the full path (HIP forward with dropout, then the HIP
backward) and keeps the plain backward's bars, relative to each exact
gradient's magnitude (which already carries keep_scale):
    max |X - X_ref| <= 2^-6 max |X_ref| + 1e-5,
    mean |X - X_ref| <= 2^-8 mean |X_ref| + 1e-6     for X in dQ, dK, dV.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import (attention_dropout_bwd_ref_rows, attention_dropout_ref, bf16_bits_to_f64,
                    f32_scale)
from tiled_attention_09_amd.synth import (WORKLOADS, bf16_bits, make_dout, make_qkv, make_workload,
                                          sample_rows)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3
MAX_REL, MEAN_REL = 2.0 ** -6, 2.0 ** -8


def _ta():
    import tiled_attention_09_amd as ta
    ta.load_library()
    return ta


def _f64(t):
    return bf16_bits_to_f64(bf16_bits(t))


def _check_fwd(q, k, v, scale, causal, seed, t, rows=None):
    ta = _ta()
    o, lse = ta.attn_fwd_dropout(q.to(DEV), k.to(DEV), v.to(DEV), seed, t, scale=scale,
                                 causal=causal)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    B, H = q.shape[:2]
    eo, el = [], []
    for b in range(B):
        for h in range(H):
            r = None if rows is None else rows[b * H + h]
            ro, rl = attention_dropout_ref(qd[b, h], kd[b, h], vd[b, h], f32_scale(scale), causal,
                                           b * H + h, seed, t, rows=r)
            sel = slice(None) if r is None else r
            eo.append(np.abs(o[b, h][sel] - ro).ravel())
            el.append(np.abs(lse[b, h][sel] - rl))
    eo, el = np.concatenate(eo), np.concatenate(el)
    ks = 256.0 / (256.0 - t)
    msg = "max|dO| %.3e mean|dO| %.3e max|dLSE| %.3e (keep_scale %.3f)" % (
        eo.max(), eo.mean(), el.max(), ks)
    print("  " + msg, flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), msg
    assert eo.max() <= O_MAX * ks and eo.mean() <= O_MEAN * ks and el.max() <= LSE_MAX, msg


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 64), (333, 64), (1003, 128)])
def test_dropout_zero_threshold_is_attn_fwd(N, d, causal):
    print("case dropout t=0 N=%d d=%d causal=%d" % (N, d, causal), flush=True)
    ta = _ta()
    q, k, v = (x.to(DEV) for x in make_qkv(2, 3, N, d, 900 + N + d))
    a = ta.attn_fwd(q, k, v, causal=causal)
    b = ta.attn_fwd_dropout(q, k, v, seed=77, drop_t=0, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("t", [26, 128, 230])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 128), (65, 64), (333, 128), (1003, 64)])
def test_dropout_forward_full_rows(N, d, causal, t):
    print("case dropout fwd N=%d d=%d causal=%d t=%d" % (N, d, causal, t), flush=True)
    q, k, v = make_qkv(2, 2, N, d, 1000 + N + d + t)
    _check_fwd(q, k, v, 1 / np.sqrt(d), causal, seed=0x1234_5678_9ABC_DEF0 + N, t=t)


def test_dropout_forward_negative_scale_large_logits():
    print("case dropout fwd negative scale", flush=True)
    q, k, v = make_qkv(1, 3, 300, 128, 1111, qk_mult=4.0)
    _check_fwd(q, k, v, -0.2, True, seed=5, t=100)


def test_dropout_masks_depend_on_seed_and_head():
    """Same inputs in every head: outputs differ between heads and seeds, and
    a repeated call reproduces its bits."""
    ta = _ta()
    q, k, v = make_qkv(1, 1, 256, 64, 1212)
    q, k, v = (x.expand(1, 2, 256, 64).contiguous().to(DEV) for x in (q, k, v))
    o1, _ = ta.attn_fwd_dropout(q, k, v, seed=1, drop_t=128)
    o1b, _ = ta.attn_fwd_dropout(q, k, v, seed=1, drop_t=128)
    o2, _ = ta.attn_fwd_dropout(q, k, v, seed=2, drop_t=128)
    torch.cuda.synchronize()
    assert torch.equal(o1, o1b)
    assert not torch.equal(o1[0, 0], o1[0, 1])
    assert not torch.equal(o1, o2)


def test_dropout_forward_headline_sampled():
    """B=2, H=32, N=8192, d=128 causal, Q,K x4, drop probability 26/256: 32
    sampled rows of every head, in the benchmark's launch configuration."""
    w = WORKLOADS["headline"]
    print("case dropout fwd headline %s" % w.describe(), flush=True)
    q, k, v = make_workload(w)
    rows = [sample_rows(w.N, 32, w.seed + 700 + i) for i in range(w.B * w.H)]
    _check_fwd(q, k, v, w.scale, w.causal, seed=2024, t=26, rows=rows)


# ---- backward ------------------------------------------------------------------

def _gpu_bwd(q, k, v, g, scale, causal, seed, t):
    ta = _ta()
    qd, kd, vd, gd = (x.to(DEV) for x in (q, k, v, g))
    o, lse = ta.attn_fwd_dropout(qd, kd, vd, seed, t, scale=scale, causal=causal)
    grads = ta.attn_bwd_dropout(qd, kd, vd, o, lse, gd, seed, t, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return tuple(x.cpu().double().numpy() for x in grads)


def _check_bwd(got, ref, what):
    msgs, ok = [], True
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        err = np.abs(a - b)
        mx, mean = np.abs(b).max(), np.abs(b).mean()
        msgs.append("%s max %.2e (rel %.2e) mean rel %.2e" % (
            name, err.max(), err.max() / max(mx, 1e-30), err.mean() / max(mean, 1e-30)))
        ok &= bool(np.all(np.isfinite(a)))
        ok &= bool(err.max() <= MAX_REL * mx + 1e-5 and err.mean() <= MEAN_REL * mean + 1e-6)
    msg = "%s: %s" % (what, "; ".join(msgs))
    print("  " + msg, flush=True)
    assert ok, msg


def _bwd_case(B, H, N, d, causal, t, seed, heads=None, qr=None, kr=None, w=None):
    scale = 1.0 / np.sqrt(d) if w is None else w.scale
    if w is None:
        q, k, v = make_qkv(B, H, N, d, seed)
        g = make_dout(B, H, N, d, seed)
    else:
        q, k, v = make_workload(w)
        g = make_dout(w.B, w.H, w.N, w.d, w.seed)
    got = _gpu_bwd(q, k, v, g, scale, causal, seed, t)
    heads = range(B * H) if heads is None else heads
    gq, gk, gv, rq, rk, rv = [], [], [], [], [], []
    for n in heads:
        b, h = divmod(n, H)
        ref = attention_dropout_bwd_ref_rows(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]),
                                             _f64(g[b, h]), f32_scale(scale), causal, n, seed, t,
                                             qr, kr)
        sq = slice(None) if qr is None else qr
        sk = slice(None) if kr is None else kr
        gq.append(got[0][b, h][sq]); gk.append(got[1][b, h][sk]); gv.append(got[2][b, h][sk])
        rq.append(ref[0]); rk.append(ref[1]); rv.append(ref[2])
    return tuple(map(np.stack, (gq, gk, gv))), tuple(map(np.stack, (rq, rk, rv)))


@pytest.mark.parametrize("t", [0, 26, 230])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 64), (65, 128), (333, 64), (1003, 128)])
def test_dropout_backward_full_rows(N, d, causal, t):
    print("case dropout bwd N=%d d=%d causal=%d t=%d" % (N, d, causal, t), flush=True)
    got, ref = _bwd_case(2, 2, N, d, causal, t, seed=3000 + N + d + t)
    _check_bwd(got, ref, "N=%d d=%d causal=%d t=%d" % (N, d, causal, t))


def test_dropout_backward_headline_sampled():
    """B=2, H=32, N=8192, d=128 causal, Q,K x4, drop probability 26/256: 64
    sampled query rows (dQ) and key rows (dK, dV) of three heads, full path."""
    w = WORKLOADS["headline"]
    print("case dropout bwd headline %s" % w.describe(), flush=True)
    got, ref = _bwd_case(w.B, w.H, w.N, w.d, w.causal, 26, seed=2025, heads=[0, 37, 63],
                         qr=sample_rows(w.N, 64, w.seed + 800),
                         kr=sample_rows(w.N, 64, w.seed + 900), w=w)
    _check_bwd(got, ref, "headline sampled")


def test_dropout_backward_deterministic():
    ta = _ta()
    B, H, N, d = 1, 3, 300, 128
    q, k, v = (x.to(DEV) for x in make_qkv(B, H, N, d, 31))
    g = make_dout(B, H, N, d, 31).to(DEV)
    o, lse = ta.attn_fwd_dropout(q, k, v, 9, 64, causal=True)
    a = ta.attn_bwd_dropout(q, k, v, o, lse, g, 9, 64, causal=True)
    b = ta.attn_bwd_dropout(q, k, v, o, lse, g, 9, 64, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.isfinite(x).all() and torch.equal(x, y)


# ---- general shapes: attn_fwd_dropout_ex / attn_bwd_dropout_ex -------------------
#
# Query row r of a chunk draws the mask row of its absolute position
# query_offset + r (the oracle's reading), so a chunk is the corresponding rows
# of the whole problem.  Same bars as above.

GENERAL_CASES = {  # name: (B, H, Nq, Nk, d, dv, offset, causal)
    "decode_step": (1, 4, 1, 1000, 128, 128, 999, True),
    "chunk_100_of_1000": (1, 3, 100, 1000, 64, 64, 900, True),
    "more_queries_than_keys": (1, 2, 300, 130, 64, 64, 0, True),
    "dv_smaller": (2, 2, 200, 333, 128, 64, 133, True),
    "dv_larger": (1, 3, 129, 257, 64, 128, 128, True),
    "cross_noncausal_ragged": (2, 2, 65, 1003, 128, 128, 0, False),
}


def _random_general(n: int, seed: int):
    """Seeded random shapes beside the named ones (the same set on every run);
    at least two keys, so the gradients do not vanish identically."""
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        nk = int(rng.integers(2, 1101))
        causal = bool(rng.integers(0, 2))
        out["random_%02d" % i] = (int(rng.integers(1, 3)), int(rng.integers(1, 4)),
                                  int(rng.integers(1, 401)), nk, int(rng.choice([64, 128])),
                                  int(rng.choice([64, 128])),
                                  int(rng.integers(0, nk + 32)) if causal else 0, causal)
    return out


GENERAL_CASES.update(_random_general(6, 9909))


def _general_inputs(B, H, Nq, Nk, d, dv, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g)
    k = torch.randn((B, H, Nk, d), generator=g)
    v = torch.randn((B, H, Nk, dv), generator=g)
    do = torch.randn((B, H, Nq, dv), generator=g)
    return tuple(x.to(torch.bfloat16).contiguous() for x in (q, k, v, do))


@pytest.mark.parametrize("t", [26, 230])
@pytest.mark.parametrize("name", sorted(GENERAL_CASES))
def test_dropout_general_forward_and_backward(name, t):
    B, H, Nq, Nk, d, dv, off, causal = GENERAL_CASES[name]
    print("case dropout general %s t=%d" % (name, t), flush=True)
    ta = _ta()
    scale, seed = 1.0 / np.sqrt(d), 4242 + Nq
    q, k, v, g = _general_inputs(B, H, Nq, Nk, d, dv, 300 + Nq + Nk)
    qd, kd, vd, gd = (x.to(DEV) for x in (q, k, v, g))
    o, lse = ta.attn_fwd_dropout_ex(qd, kd, vd, seed, t, scale=scale, causal=causal,
                                    query_offset=off)
    grads = ta.attn_bwd_dropout_ex(qd, kd, vd, o, lse, gd, seed, t, scale=scale, causal=causal,
                                   query_offset=off)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    got = tuple(x.cpu().double().numpy() for x in grads)
    eo, el, rq, rk, rv = [], [], [], [], []
    for b in range(B):
        for h in range(H):
            n = b * H + h
            args = (_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]))
            ro, rl = attention_dropout_ref(*args, f32_scale(scale), causal, n, seed, t,
                                           query_offset=off)
            eo.append(np.abs(o[b, h] - ro).ravel())
            el.append(np.abs(lse[b, h] - rl))
            ref = attention_dropout_bwd_ref_rows(*args, _f64(g[b, h]), f32_scale(scale), causal, n,
                                                 seed, t, query_offset=off)
            rq.append(ref[0]); rk.append(ref[1]); rv.append(ref[2])
    eo, el = np.concatenate(eo), np.concatenate(el)
    ks = 256.0 / (256.0 - t)
    msg = "max|dO| %.3e mean|dO| %.3e max|dLSE| %.3e" % (eo.max(), eo.mean(), el.max())
    print("  " + msg, flush=True)
    assert eo.max() <= O_MAX * ks and eo.mean() <= O_MEAN * ks and el.max() <= LSE_MAX, msg
    ref = tuple(np.stack(x).reshape(B, H, *x[0].shape) for x in (rq, rk, rv))
    _check_bwd(got, ref, "general dropout backward")


def test_dropout_general_zero_threshold_is_attn_fwd_ex():
    ta = _ta()
    q, k, v, _ = (x.to(DEV) for x in _general_inputs(1, 3, 100, 1000, 64, 128, 77))
    a = ta.attn_fwd_ex(q, k, v, causal=True, query_offset=900)
    b = ta.attn_fwd_dropout_ex(q, k, v, 5, 0, causal=True, query_offset=900)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_dropout_chunk_is_rows_of_the_square_problem():
    """Queries 640..767 of a square causal problem run as a chunk at offset 640
    give the same rows as the square dropout forward (same seed, same mask)."""
    ta = _ta()
    q, k, v = (x.to(DEV) for x in make_qkv(1, 2, 1000, 128, 78))
    full = ta.attn_fwd_dropout(q, k, v, 99, 64, causal=True)
    part = ta.attn_fwd_dropout_ex(q[:, :, 640:768].contiguous(), k, v, 99, 64, causal=True,
                                  query_offset=640)
    torch.cuda.synchronize()
    do = (part[0] - full[0][:, :, 640:768]).abs().max().item()
    dl = (part[1] - full[1][:, :, 640:768]).abs().max().item()
    print("  chunk vs square rows: max|dO| %.2e max|dLSE| %.2e" % (do, dl), flush=True)
    assert do <= 1e-5 and dl <= 1e-6
