"""GPU parity of the FP8 path: the per-head quantiser (bit-exact codes and
descales against the oracle's float32 recipe) and the FP8-score forward
(against the float64 oracle evaluated on the oracle's own codes).

Bars: max |dO| <= 1e-2 and mean |dO| <= 1e-3 (the bf16 forward's), and per
row |dLSE_i| <= 1e-3 + 2^-14 * max_j |S_ij|.  Both sides see the same
quantised Q and K (the codes are checked equal first).  The LSE bar is wider
than the bf16 path's because the FP8 32x32x64 matrix instruction sums its
products internally at about 21 significant bits (measured: 63 terms of 2^-6
added to 448^2 lose 0.109; random E4M3 codes: error up to 3.2e-5 of the
largest result), so a score S carries an error of order 2^-15 |S|, and LSE,
a smooth maximum of the scores, moves by at most the largest score error.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention_ref, bf16_bits_to_f64, e4m3_decode, f32_scale, quantize_per_head
from tiled_attention_09_amd.synth import WORKLOADS, bf16_bits, make_qkv, make_workload, sample_rows

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3


def _ta():
    import tiled_attention_09_amd as ta
    ta.load_library()
    return ta


def _f64(t):
    return bf16_bits_to_f64(bf16_bits(t))


@pytest.mark.parametrize("case", ["normal", "x4", "tiny", "zero_head", "d64", "ragged"])
def test_quantizer_bit_exact(case):
    shape = {"d64": (2, 3, 333, 64), "ragged": (1, 5, 77, 128)}.get(case, (2, 3, 333, 128))
    g = torch.Generator().manual_seed(40 + len(case))
    x = torch.randn(shape, generator=g)
    if case == "x4":
        x *= 4
    if case == "tiny":
        x *= 2.0 ** -12                      # exercises E4M3 subnormal codes after scaling
    if case == "zero_head":
        x[1, 1] = 0
    x = x.to(torch.bfloat16).contiguous()
    print("case quantizer %s %s" % (case, tuple(shape)), flush=True)
    codes, descale = _ta().attn_quantize_fp8(x.to(DEV))
    torch.cuda.synchronize()
    rc, rd = quantize_per_head(_f64(x))
    got_c, got_d = codes.cpu().numpy(), descale.cpu().numpy()
    n_diff = int(np.sum(got_c != rc))
    print("  codes differing: %d of %d; descales equal: %s" % (n_diff, rc.size,
                                                               np.array_equal(got_d, rd)), flush=True)
    assert n_diff == 0
    assert np.array_equal(got_d, rd)


def _fp8_case(q, k, v, scale, causal, rows=None):
    """Returns (|dO| values, |dLSE| per row, LSE bar per row)."""
    ta = _ta()
    q8, qd = ta.attn_quantize_fp8(q.to(DEV))
    k8, kd = ta.attn_quantize_fp8(k.to(DEV))
    o, lse = ta.attn_fwd_fp8(q8, k8, v.to(DEV), qd, kd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    rq8, rqd = quantize_per_head(_f64(q))
    rk8, rkd = quantize_per_head(_f64(k))
    assert np.array_equal(q8.cpu().numpy(), rq8) and np.array_equal(k8.cpu().numpy(), rk8)
    qf = e4m3_decode(rq8) * rqd[..., None, None].astype(np.float64)
    kf = e4m3_decode(rk8) * rkd[..., None, None].astype(np.float64)
    vf = _f64(v)
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    B, H = q.shape[:2]
    errs_o, errs_l, bars = [], [], []
    for b in range(B):
        for h in range(H):
            r = rows[b * H + h] if rows is not None else None
            ro, rl = attention_ref(qf[b, h], kf[b, h], vf[b, h], f32_scale(scale), causal, rows=r)
            sel = slice(None) if r is None else r
            ridx = np.arange(q.shape[2]) if r is None else r
            sc = f32_scale(scale) * (qf[b, h][ridx] @ kf[b, h].T)
            if causal:
                sc = np.where(np.arange(sc.shape[1])[None, :] > ridx[:, None], 0.0, sc)
            bars.append(1e-3 + 2.0 ** -14 * np.abs(sc).max(axis=1))
            errs_o.append(np.abs(o[b, h][sel] - ro).ravel())
            errs_l.append(np.abs(lse[b, h][sel] - rl))
    return np.concatenate(errs_o), np.concatenate(errs_l), np.concatenate(bars)


def _check(do, dl, bar):
    msg = "max|dO| %.3e mean|dO| %.3e max|dLSE| %.3e (worst dLSE/bar %.2f)" % (
        do.max(), do.mean(), dl.max(), (dl / bar).max())
    print("  " + msg, flush=True)
    assert do.max() <= O_MAX and do.mean() <= O_MEAN and np.all(dl <= bar), msg


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,mult", [(1, 1.0), (65, 1.0), (333, 1.0), (1003, 4.0)])
def test_fp8_forward_full_rows(N, mult, causal):
    print("case fp8 fwd N=%d mult=%g causal=%d" % (N, mult, causal), flush=True)
    q, k, v = make_qkv(2, 2, N, 128, 70 + N, mult)
    _check(*_fp8_case(q, k, v, 1 / np.sqrt(128), causal))


def test_fp8_forward_headline_sampled():
    """B=2, H=32, N=8192, d=128 causal, Q,K x4: 128 sampled rows of every head."""
    w = WORKLOADS["headline"]
    print("case fp8 fwd headline %s" % w.describe(), flush=True)
    q, k, v = make_workload(w)
    rows = [sample_rows(w.N, 128, w.seed + 500 + i) for i in range(w.B * w.H)]
    _check(*_fp8_case(q, k, v, w.scale, w.causal, rows=rows))


def test_fp8_negative_scale_and_descale_folding():
    """A negative scale and heads with very different magnitudes (descales)."""
    q, k, v = make_qkv(1, 3, 300, 128, 81)
    q[0, 0] *= 16
    k[0, 2] *= 2.0 ** -6
    _check(*_fp8_case(q.contiguous(), k.contiguous(), v, -0.2, True))
