"""GPU parity of the HIP attention backward against the float64 oracle.

Same seeded bf16 inputs (Q, K, V and the output gradient G) on both sides.
Two ways in:
  * isolated: the kernels get the oracle's O and LSE (rounded to float32), so
    only the backward's own arithmetic is measured;
  * full path: the kernels get the HIP forward's O and LSE, as a user runs it.
The oracle always computes the gradients from its own exact probabilities.

Bar, per gradient tensor X in {dQ, dK, dV} (float32 outputs):
    max |X - X_ref|  <= 2^-6 max |X_ref| + 1e-5
    mean |X - X_ref| <= 2^-8 mean |X_ref| + 1e-6
(the absolute floors only matter where the exact gradient is zero, e.g. dQ and
dK of a single key)
Every product term on the GPU carries one bf16 rounding of P or dS (relative
2^-9) and fp32 accumulation; the full path adds the forward's O and LSE errors
through D and the rebuilt P.  Small shapes are compared on every row; the two
large workloads on sampled query rows (dQ) and key rows (dK, dV) of a few
heads, in the launch configuration the benchmark times.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import (attention_bwd_ref_batched, attention_ref_batched, bf16_bits_to_f64,
                    f32_scale)
from tiled_attention_09_amd.synth import (WORKLOADS, bf16_bits, make_dout, make_qkv,
                                          make_workload, sample_rows)

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL = 2.0 ** -6, 2.0 ** -8
DEV = torch.device("cuda:0")


def _ta():
    import tiled_attention_09_amd as ta
    ta.load_library()
    return ta


def _f64(t):
    return bf16_bits_to_f64(bf16_bits(t))


def _gpu_bwd(q, k, v, g, scale, causal, o=None, lse=None):
    """Gradients from the HIP path; O and LSE from the HIP forward unless given."""
    ta = _ta()
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    if o is None:
        o, lse = ta.attn_fwd(qd, kd, vd, scale=scale, causal=causal)
    else:
        o, lse = o.to(DEV), lse.to(DEV)
    dq, dk, dv = ta.attn_bwd(qd, kd, vd, o, lse, gd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return tuple(x.cpu().double().numpy() for x in (dq, dk, dv))


def _check(got, ref, what):
    msgs, ok = [], True
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        err = np.abs(a - b)
        mx, mean = np.abs(b).max(), np.abs(b).mean()
        msgs.append("%s max %.2e (rel %.2e) mean rel %.2e" % (
            name, err.max(), err.max() / max(mx, 1e-30), err.mean() / max(mean, 1e-30)))
        ok &= bool(np.all(np.isfinite(a)))
        ok &= bool(err.max() <= MAX_REL * mx + 1e-5 and err.mean() <= MEAN_REL * mean + 1e-6)
    msg = "%s: %s" % (what, "; ".join(msgs))
    print(msg, flush=True)
    assert ok, msg


def _oracle_o_lse(q, k, v, scale, causal):
    o, lse = attention_ref_batched(_f64(q), _f64(k), _f64(v), f32_scale(scale), causal)
    return torch.from_numpy(o).float().contiguous(), torch.from_numpy(lse).float().contiguous()


def _full_case(B, H, N, d, causal, seed, isolated, qk_mult=1.0):
    scale = 1.0 / np.sqrt(d)
    q, k, v = make_qkv(B, H, N, d, seed, qk_mult)
    g = make_dout(B, H, N, d, seed)
    o = lse = None
    if isolated:
        o, lse = _oracle_o_lse(q, k, v, scale, causal)
    got = _gpu_bwd(q, k, v, g, scale, causal, o, lse)
    ref = attention_bwd_ref_batched(_f64(q), _f64(k), _f64(v), _f64(g), f32_scale(scale), causal)
    ref = tuple(r.reshape(B, H, N, d) for r in ref)
    return got, ref


@pytest.mark.parametrize("isolated", [True, False], ids=["isolated", "full_path"])
@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_workload_full_rows(name, isolated):
    w = WORKLOADS[name]
    print("case bwd %s %s %s" % (name, w.describe(), "isolated" if isolated else "full"),
          flush=True)
    got, ref = _full_case(w.B, w.H, w.N, w.d, w.causal, w.seed, isolated, w.qk_mult)
    _check(got, ref, name)


@pytest.mark.parametrize("isolated", [True, False], ids=["isolated", "full_path"])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_mid(d, isolated):
    print("case bwd causal B=2,H=3,N=700,d=%d" % d, flush=True)
    got, ref = _full_case(2, 3, 700, d, True, 11 + d, isolated)
    _check(got, ref, "causal N=700 d=%d" % d)


@pytest.mark.parametrize("d", [64, 128])
def test_causal_eight_heads_few_tiles(d):
    # 8 heads and 6 tiles per head: the dQ and dK/dV grids take the XCDs'
    # tiles longest first across heads (the order used below 64 / 32 tiles).
    print("case bwd causal B=2,H=4,N=700,d=%d" % d, flush=True)
    got, ref = _full_case(2, 4, 700, d, True, 31 + d, False)
    _check(got, ref, "causal B=2,H=4,N=700 d=%d" % d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 31, 33, 63, 64, 65, 127, 128, 129, 191, 255, 257])
def test_edge_lengths(N, d, causal):
    print("case bwd edge N=%d d=%d causal=%d" % (N, d, causal), flush=True)
    got, ref = _full_case(1, 2, N, d, causal, 1000 + N, True)
    _check(got, ref, "N=%d d=%d causal=%d" % (N, d, causal))


@pytest.mark.parametrize("name,heads", [("headline", [0, 37, 63]), ("long", [9])])
def test_workload_sampled_rows(name, heads):
    """Full-size workloads: HIP forward then HIP backward (the timed path);
    gradients of sampled rows of a few heads against the oracle."""
    w = WORKLOADS[name]
    print("case bwd %s %s sampled heads %s" % (name, w.describe(), heads), flush=True)
    q, k, v = make_workload(w)
    g = make_dout(w.B, w.H, w.N, w.d, w.seed)
    got = _gpu_bwd(q, k, v, g, w.scale, w.causal)
    qr = sample_rows(w.N, 64, w.seed + 300)
    kr = sample_rows(w.N, 64, w.seed + 400)
    sel = [(f // w.H, f % w.H) for f in heads]
    sub = lambda t: torch.stack([t[b, h] for b, h in sel])[None]     # [1, nh, N, d]
    ref = attention_bwd_ref_batched(_f64(sub(q)), _f64(sub(k)), _f64(sub(v)), _f64(sub(g)),
                                    f32_scale(w.scale), w.causal, query_rows=qr, key_rows=kr)
    gq = np.stack([got[0][b, h][qr] for b, h in sel])
    gk = np.stack([got[1][b, h][kr] for b, h in sel])
    gv = np.stack([got[2][b, h][kr] for b, h in sel])
    _check((gq, gk, gv), ref, "%s sampled" % name)


def test_deterministic_and_every_row_written():
    ta = _ta()
    B, H, N, d = 2, 2, 333, 128
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, N, d, 77))
    g = make_dout(B, H, N, d, 77).to(DEV)
    o, lse = ta.attn_fwd(q, k, v, causal=True)
    outs = []
    for fill in (float("nan"), 0.0):
        grads = tuple(torch.full((B, H, N, d), fill, device=DEV) for _ in range(3))
        ws = torch.full((ta.attn_bwd_workspace_size(B, H, N),), 255, dtype=torch.uint8, device=DEV)
        outs.append(ta.attn_bwd(q, k, v, o, lse, g, causal=True, grads=grads, workspace=ws))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)


def test_zero_scale_closed_form():
    """scale = 0: uniform weights over visible keys, dQ = dK = 0 exactly and
    dV[j] = sum over queries i >= j of G[i] / (i + 1)."""
    B, H, N, d = 1, 2, 200, 64
    q, k, v = make_qkv(B, H, N, d, 5)
    g = make_dout(B, H, N, d, 5)
    dq, dk, dv = _gpu_bwd(q, k, v, g, 0.0, True)
    assert np.all(dq == 0) and np.all(dk == 0)
    gg = _f64(g)
    w = np.tril(1.0 / np.arange(1, N + 1)[:, None] * np.ones((N, N)))
    ref = np.einsum("ij,bhic->bhjc", w, gg)
    err = np.abs(dv - ref).max()
    print("zero scale dV max err %.2e" % err, flush=True)
    assert err <= 2.0 ** -8 * np.abs(ref).max()


def test_single_key():
    """N = 1: P = 1, so dQ = dK = 0 up to rounding and dV = G."""
    q, k, v = make_qkv(3, 2, 1, 128, 6)
    g = make_dout(3, 2, 1, 128, 6)
    dq, dk, dv = _gpu_bwd(q, k, v, g, 1 / np.sqrt(128), False)
    assert np.abs(dq).max() < 1e-4 and np.abs(dk).max() < 1e-4
    np.testing.assert_allclose(dv, _f64(g), rtol=0, atol=1e-2)


def test_head_isolation():
    """NaN inputs in one head leave the neighbouring heads' gradients intact."""
    B, H, N, d = 1, 3, 130, 64
    q, k, v = make_qkv(B, H, N, d, 8)
    g = make_dout(B, H, N, d, 8)
    for t in (q, k, v, g):
        t[0, 0] = float("nan")
        t[0, 2] = float("nan")
    got = _gpu_bwd(q, k, v, g, 0.125, False)
    q1, k1, v1, g1 = (t[:, 1:2].contiguous() for t in (q, k, v, g))
    ref = attention_bwd_ref_batched(_f64(q1), _f64(k1), _f64(v1), _f64(g1), 0.125, False)
    _check(tuple(x[0, 1][None] for x in got), ref, "middle head")


def test_negative_scale_large_logits():
    B, H, N, d = 1, 2, 300, 128
    q, k, v = make_qkv(B, H, N, d, 9, qk_mult=4.0)
    g = make_dout(B, H, N, d, 9)
    o, lse = _oracle_o_lse(q, k, v, -0.125, True)
    got = _gpu_bwd(q, k, v, g, -0.125, True, o, lse)
    ref = attention_bwd_ref_batched(_f64(q), _f64(k), _f64(v), _f64(g), -0.125, True)
    _check(got, tuple(r.reshape(B, H, N, d) for r in ref), "negative scale x4 logits")


def test_side_stream():
    ta = _ta()
    B, H, N, d = 1, 2, 256, 64
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, N, d, 10))
    g = make_dout(B, H, N, d, 10).to(DEV)
    o, lse = ta.attn_fwd(q, k, v)
    ref = ta.attn_bwd(q, k, v, o, lse, g)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = ta.attn_bwd(q, k, v, o, lse, g)
    s.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
