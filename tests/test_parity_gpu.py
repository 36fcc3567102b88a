"""GPU parity: the HIP attention forward against the float64 oracle.

Same seeded bf16 inputs on both sides.  Bar (fp32 O and LSE):
    max |O - O_ref| <= 1e-2,  mean |O - O_ref| <= 1e-3,  max |LSE - LSE_ref| <= 1e-3.
Small workloads are compared on every row; the two large ones on 256 sampled
query rows per head (fixed tile-edge rows plus a seeded fill), in the same
launch configuration the benchmark times.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import attention_ref, attention_ref_batched, bf16_bits_to_f64, f32_scale
from tiled_attention_09_amd.synth import WORKLOADS, bf16_bits, make_qkv, make_workload, sample_rows

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3


def _ta():
    import tiled_attention_09_amd as ta
    ta.load_library()
    return ta


def _f64(t):
    return bf16_bits_to_f64(bf16_bits(t))


def _run(q, k, v, scale, causal):
    ta = _ta()
    dev = torch.device("cuda:0")
    o, lse = ta.attn_fwd(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def _check(o, lse, ro, rl, what):
    do = np.abs(o - ro)
    dl = np.abs(lse - rl)
    msg = "%s: max|dO| %.3e mean|dO| %.3e max|dLSE| %.3e" % (what, do.max(), do.mean(), dl.max())
    print(msg, flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), msg
    assert do.max() <= O_MAX and do.mean() <= O_MEAN and dl.max() <= LSE_MAX, msg


@pytest.mark.parametrize("name", ["tiny", "ragged", "mid_causal"])
def test_workload_full_rows(name):
    w = WORKLOADS[name]
    print("case %s %s" % (name, w.describe()), flush=True)
    q, k, v = make_workload(w)
    o, lse = _run(q, k, v, w.scale, w.causal)
    ro, rl = attention_ref_batched(_f64(q), _f64(k), _f64(v), f32_scale(w.scale), w.causal)
    _check(o, lse, ro, rl, name)


@pytest.mark.parametrize("name", ["headline", "long"])
def test_workload_sampled_rows(name):
    w = WORKLOADS[name]
    print("case %s %s" % (name, w.describe()), flush=True)
    q, k, v = make_workload(w)
    o, lse = _run(q, k, v, w.scale, w.causal)
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    s = f32_scale(w.scale)
    errs_o, errs_l = [], []
    for b in range(w.B):
        for h in range(w.H):
            rows = sample_rows(w.N, 256, w.seed + 100 + b * w.H + h)
            ro, rl = attention_ref(qd[b, h], kd[b, h], vd[b, h], s, w.causal, rows=rows)
            errs_o.append(np.abs(o[b, h, rows] - ro))
            errs_l.append(np.abs(lse[b, h, rows] - rl))
    do = np.concatenate([e.ravel() for e in errs_o])
    dl = np.concatenate(errs_l)
    msg = "%s sampled: max|dO| %.3e mean|dO| %.3e max|dLSE| %.3e" % (name, do.max(), do.mean(),
                                                                    dl.max())
    print(msg, flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert do.max() <= O_MAX and do.mean() <= O_MEAN and dl.max() <= LSE_MAX, msg


EDGE_N = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257, 1003]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths_against_oracle(d, causal):
    """Lengths around wave, tile and workgroup boundaries (and the page's 1003)."""
    for n in EDGE_N:
        q, k, v = make_qkv(2, 3, n, d, seed=1000 + n + d + causal)
        o, lse = _run(q, k, v, 1 / math.sqrt(d), causal)
        ro, rl = attention_ref_batched(_f64(q), _f64(k), _f64(v), f32_scale(1 / math.sqrt(d)), causal)
        _check(o, lse, ro, rl, "N=%d d=%d causal=%d" % (n, d, causal))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_closed_forms(d, causal):
    """scale 0 gives the (prefix) mean of V and LSE = ln(count); one key gives V_0;
    constant V returns V."""
    for n in (1, 65, 200):
        q, k, v = make_qkv(1, 2, n, d, seed=77 + n)
        vd = _f64(v)
        o, lse = _run(q, k, v, 0.0, causal)
        counts = np.arange(1, n + 1) if causal else np.full(n, n)
        mean = np.cumsum(vd, axis=2) / counts[:, None] if causal else np.repeat(
            vd.mean(axis=2, keepdims=True), n, axis=2)
        _check(o, lse, mean, np.broadcast_to(np.log(counts), lse.shape), "scale0 N=%d" % n)
        c = torch.randn(d, generator=torch.Generator().manual_seed(n)).to(torch.bfloat16)
        vc = c.expand(1, 2, n, d).contiguous()
        o, _ = _run(q, k, vc, 1 / math.sqrt(d), causal)
        # P enters the value product rounded to bf16 while l sums the fp32 p, so
        # O = c * sum(bf16(p)) / sum(p): relative error at most 2^-9.
        cd = _f64(c)
        assert np.max(np.abs(o - cd[None, None, None, :])) <= 2.0 ** -8 * np.abs(cd).max()
    q, k, v = make_qkv(1, 1, 1, d, seed=5)
    o, lse = _run(q, k, v, 0.3, causal)
    assert np.max(np.abs(o - _f64(v))) <= 1e-6
    ref = f32_scale(0.3) * float((_f64(q)[0, 0, 0] * _f64(k)[0, 0, 0]).sum())
    assert abs(lse[0, 0, 0] - ref) <= 1e-4


@pytest.mark.parametrize("first_big", [False, True])
def test_worked_example_two_tiles(first_big):
    """Scores 1000 and 1001 land in different key tiles (page "22. GPU
    Engineering", sec. 22.7): the first contribution must be rescaled by e^-1.
    Every query is e0 + e1; key 0 = 1000 e0, key 64 = 1000 e0 + e1 (exact in
    bf16), all other keys -1000 e0."""
    d, n = 64, 128
    q = torch.zeros(1, 1, n, d)
    q[..., 0] = 1.0
    q[..., 1] = 1.0
    k = torch.zeros(1, 1, n, d)
    k[..., 0] = -1000.0
    a, b = (64, 0) if first_big else (0, 64)
    k[0, 0, a, 0] = 1000.0
    k[0, 0, b, 0] = 1000.0
    k[0, 0, b, 1] = 1.0
    v = torch.randn(1, 1, n, d, generator=torch.Generator().manual_seed(3))
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    o, lse = _run(q, k, v, 1.0, False)
    vd = _f64(v)[0, 0]
    e = math.exp(-1.0)
    want = (e * vd[a] + vd[b]) / (1 + e)
    # without the rescale the first key would weigh 1, not e^-1: an error near 0.5|v|
    assert np.max(np.abs(o[0, 0] - want[None, :])) <= O_MAX
    assert np.max(np.abs(lse[0, 0] - (1001.0 + math.log1p(e)))) <= LSE_MAX


def test_deterministic_and_every_row_written():
    ta = _ta()
    w = WORKLOADS["ragged"]
    q, k, v = (x.cuda() for x in make_workload(w))
    o1 = torch.full((w.B, w.H, w.N, w.d), float("nan"), device="cuda")
    l1 = torch.full((w.B, w.H, w.N), float("nan"), device="cuda")
    ta.attn_fwd(q, k, v, w.scale, w.causal, out=o1, lse=l1)
    o2, l2 = ta.attn_fwd(q, k, v, w.scale, w.causal)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_heads_are_isolated():
    """A ragged head never reads its neighbour: NaN in head 1 leaves head 0 clean."""
    q, k, v = make_qkv(1, 2, 1003, 64, seed=9)
    k[0, 1] = float("nan")
    v[0, 1] = float("nan")
    o, lse = _run(q, k, v, 0.125, False)
    assert np.all(np.isfinite(o[0, 0])) and np.all(np.isfinite(lse[0, 0]))
    ro, rl = attention_ref(_f64(q)[0, 0], _f64(k)[0, 0], _f64(v)[0, 0], 0.125, False)
    _check(o[0, 0], lse[0, 0], ro, rl, "isolated head")


def test_negative_scale_and_large_logits():
    q, k, v = make_qkv(1, 2, 300, 128, seed=21, qk_mult=4.0)
    for scale in (-0.2, 0.5):
        o, lse = _run(q, k, v, scale, True)
        ro, rl = attention_ref_batched(_f64(q), _f64(k), _f64(v), f32_scale(scale), True)
        _check(o, lse, ro, rl, "scale=%g" % scale)


def test_stream_argument():
    ta = _ta()
    q, k, v = (x.cuda() for x in make_qkv(1, 2, 256, 64, seed=4))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = ta.attn_fwd(q, k, v, causal=True)
    s.synchronize()
    ro, rl = attention_ref_batched(_f64(q.cpu()), _f64(k.cpu()), _f64(v.cpu()), f32_scale(0.125), True)
    _check(o.cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl, "side stream")
