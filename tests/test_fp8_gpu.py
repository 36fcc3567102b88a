"""GPU parity of the FP8 path: the per-head quantiser (bit-exact codes and
descales against the oracle's float32 recipe), the FP8-score forward (against
the float64 oracle evaluated on the oracle's own codes) and the precision of
the FP8 score product itself.  Head dims 64 and 128 (one or two 32x32x64
products per 32 keys).

Bars: max |dO| <= 1e-2 and mean |dO| <= 1e-3 (the bf16 forward's), and per
row |dLSE_i| <= 1e-3 + 2^-11 * max_j G_ij, where G_ij bounds the score
product's own rounding.  The 32x32x64 FP8 matrix instruction sums its 64
products at less than float32 precision, with an error that scales with the
largest product of the block: test_fp8_score_product_precision pins
|dS_ij| <= 2^-11 sum_b max_{k in b} |q8_ik k8_jk| (b: the 64-term blocks of
the head dim) on constructed and 1024 random code vectors per head dim
against the exact sums (measured: 2^-11.6 at worst over 12288 random vectors
of uniform codes; quantised gaussians stay below 2^-12.6).  In the forward
tests max_{k in b} |q_ik k_jk| is bounded by max_{k in b} |q_ik| times
max_{k in b} |k_jk| (descales and scale included), which gives G.  LSE, a
smooth maximum of a row's scores, moves by at most the largest score error;
1e-3 covers the float32 softmax itself.  Both sides see the same quantised Q
and K (the codes are checked equal first).
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
SCORE_TOL = 2.0 ** -11   # |dS_ij| <= SCORE_TOL * sum_b max_{k in b} |q_ik k_jk| (pinned below)


def _ta():
    import tiled_attention_09_amd as ta
    ta.load_library()
    return ta


def _f64(t):
    return bf16_bits_to_f64(bf16_bits(t))


def _lse_bar(qf, kf, scale, visible=None):
    """Per-row LSE bar 1e-3 + SCORE_TOL * max_j G_ij for float64 Q [n, d] and
    K [m, d] (descales applied), G_ij = |scale| sum_b max_{k in b} |q_ik|
    max_{k in b} |k_jk| over the 64-wide blocks b; visible: [n, m] bool or None."""
    d = qf.shape[1]
    g = np.zeros((qf.shape[0], kf.shape[0]))
    for b in range(0, d, 64):
        g += np.outer(np.abs(qf[:, b:b + 64]).max(axis=1), np.abs(kf[:, b:b + 64]).max(axis=1))
    g *= abs(f32_scale(scale))
    if visible is not None:
        g = np.where(visible, g, 0.0)
    return 1e-3 + SCORE_TOL * g.max(axis=1)


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
            vis = (np.arange(kf.shape[2])[None, :] <= ridx[:, None]) if causal else None
            bars.append(_lse_bar(qf[b, h][ridx], kf[b, h], scale, vis))
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


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,mult", [(1, 1.0), (65, 1.0), (1003, 4.0), (2100, 1.0)])
def test_fp8_forward_d64(N, mult, causal):
    """d = 64: rows of 64 codes, one 32x32x64 product per 32 keys."""
    print("case fp8 fwd d=64 N=%d mult=%g causal=%d" % (N, mult, causal), flush=True)
    q, k, v = make_qkv(2, 3, N, 64, 170 + N, mult)
    _check(*_fp8_case(q, k, v, 1 / np.sqrt(64), causal))


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


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_negative_descales(causal, d):
    """Caller-supplied descales of either sign: head 0 has a negative Q descale,
    head 1 a negative K descale, head 2 both (a positive product).  With a
    positive scale the instance takes the row maximum on raw scores; a negative
    descale product must be folded in exactly, not give a wrong maximum."""
    ta = _ta()
    q, k, v = make_qkv(1, 3, 333, d, 91, 4.0)
    print("case fp8 negative descales causal=%d d=%d" % (causal, d), flush=True)
    q8, qd = ta.attn_quantize_fp8(q.to(DEV))
    k8, kd = ta.attn_quantize_fp8(k.to(DEV))
    sign_q = torch.tensor([[-1.0, 1.0, -1.0]], device=DEV)
    sign_k = torch.tensor([[1.0, -1.0, -1.0]], device=DEV)
    qd_s, kd_s = (qd * sign_q).contiguous(), (kd * sign_k).contiguous()
    scale = 1 / np.sqrt(d)
    o, lse = ta.attn_fwd_fp8(q8, k8, v.to(DEV), qd_s, kd_s, scale=scale, causal=causal)
    torch.cuda.synchronize()
    rq8, rqd = quantize_per_head(_f64(q))
    rk8, rkd = quantize_per_head(_f64(k))
    qf = e4m3_decode(rq8) * (rqd * sign_q.cpu().numpy())[..., None, None]
    kf = e4m3_decode(rk8) * (rkd * sign_k.cpu().numpy())[..., None, None]
    vf = _f64(v)
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    errs_o, errs_l, bars = [], [], []
    for h in range(3):
        ro, rl = attention_ref(qf[0, h], kf[0, h], vf[0, h], f32_scale(scale), causal)
        n = qf.shape[2]
        vis = np.tril(np.ones((n, n), dtype=bool)) if causal else None
        bars.append(_lse_bar(qf[0, h], kf[0, h], scale, vis))
        errs_o.append(np.abs(o[0, h] - ro).ravel())
        errs_l.append(np.abs(lse[0, h] - rl))
    _check(np.concatenate(errs_o), np.concatenate(errs_l), np.concatenate(bars))


# ---- precision of the FP8 score product itself ----------------------------------
#
# With one key per head (N = 1), unit descales and scale 1, a row's LSE is its
# single score S = <q8, k8> (the kernel forms LSE = (m c) ln 2 with m the
# product's output and c = log2 e in float32: relative rounding below 2^-21).
# Products of E4M3 values need at most 8 significant bits and a 128-term sum
# at most 43, so float64 gives the exact S.  The rounding inside the 32x32x64
# FP8 instruction is bounded relative to the largest product of its 64-term
# block (terms can cancel, so |S| is no scale for it), and the blocks of a
# d = 128 row add their errors through the float32 accumulator.


def _code_cases(n_random=1024):
    """Code vector pairs (128 codes each; d = 64 uses the first 64): structured
    sums, then random codes over the whole finite E4M3 range and over a
    narrower exponent band (half each)."""
    rng = np.random.default_rng(1234)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(np.arange(256, dtype=np.uint8))
    code_of = {float(v): c for c, v in enumerate(vals) if np.isfinite(v) and c < 0x80}
    cases = []
    # 448^2 plus 63 products of 2^-3 * 2^-3 = 2^-6 in the same 64-term block.
    q = np.zeros(128, np.uint8); k = np.zeros(128, np.uint8)
    q[0] = k[0] = code_of[448.0]
    q[1:64] = k[1:64] = code_of[0.125]
    cases.append((q, k))
    # The same small terms in the second block (accumulated through the first's output).
    q = np.zeros(128, np.uint8); k = np.zeros(128, np.uint8)
    q[0] = k[0] = code_of[448.0]
    q[64:127] = k[64:127] = code_of[0.125]
    cases.append((q, k))
    # Exact cancellation: +448^2 and -448^2, and a large cancelling pair with a tail.
    q = np.zeros(128, np.uint8); k = np.zeros(128, np.uint8)
    q[0] = q[1] = code_of[448.0]; k[0] = code_of[448.0]; k[1] = code_of[448.0] | 0x80
    cases.append((q, k))
    q = np.zeros(128, np.uint8); k = np.zeros(128, np.uint8)
    q[0] = q[70] = code_of[448.0]; k[0] = code_of[448.0]; k[70] = code_of[448.0] | 0x80
    q[5:9] = k[5:9] = code_of[1.0]
    cases.append((q, k))
    # Every term the same (a long run of equal products).
    cases.append((np.full(128, code_of[3.0], np.uint8), np.full(128, code_of[5.0], np.uint8)))
    n_struct = len(cases)
    while len(cases) < n_struct + n_random // 2:
        cases.append((rng.choice(finite, 128), rng.choice(finite, 128)))
    band = np.array([c for c in finite if 0.25 <= abs(vals[c]) <= 64.0], dtype=np.uint8)
    while len(cases) < n_struct + n_random:
        cases.append((rng.choice(band, 128), rng.choice(band, 128)))
    return cases


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_score_product_precision(d):
    ta = _ta()
    cases = _code_cases()
    H = len(cases)
    q8 = np.stack([c[0][:d] for c in cases]).reshape(1, H, 1, d)
    k8 = np.stack([c[1][:d] for c in cases]).reshape(1, H, 1, d)
    print("case fp8 score product precision d=%d: %d constructed single-key heads" % (d, H),
          flush=True)
    v = torch.ones((1, H, 1, d), dtype=torch.bfloat16, device=DEV)
    ones = torch.ones((1, H), dtype=torch.float32, device=DEV)
    _, lse = ta.attn_fwd_fp8(torch.from_numpy(q8).to(DEV), torch.from_numpy(k8).to(DEV), v, ones,
                             ones, scale=1.0, causal=False)
    torch.cuda.synchronize()
    got = lse.cpu().double().numpy().reshape(H)
    terms = e4m3_decode(q8.reshape(H, d)) * e4m3_decode(k8.reshape(H, d))
    exact = terms.sum(axis=1)
    gmax = sum(np.abs(terms[:, b:b + 64]).max(axis=1) for b in range(0, d, 64))
    err = np.abs(got - exact)
    rel = err / np.maximum(gmax, 1e-300)
    print("  max |dS| / sum of block maxima = %.3e (2^%.1f); structured cases: %s" % (
        rel.max(), np.log2(max(rel.max(), 1e-300)), ["%.2e" % x for x in rel[:5]]), flush=True)
    assert np.all(err <= SCORE_TOL * gmax + 2.0 ** -21 * np.abs(exact)), rel.max()


# ---- general shapes: attn_fwd_fp8_ex ----------------------------------------------

FP8_GENERAL = {  # name: (B, H, Nq, Nk, d, dv, offset, causal, mult)
    "decode_step": (1, 4, 1, 1000, 128, 128, 999, True, 1.0),
    "chunk_100_of_1000": (1, 3, 100, 1000, 128, 128, 900, True, 4.0),
    "more_queries_than_keys": (1, 2, 300, 130, 128, 128, 0, True, 1.0),
    "dv64": (2, 2, 200, 333, 128, 64, 133, True, 1.0),
    "cross_noncausal_ragged": (2, 2, 65, 1003, 128, 128, 0, False, 1.0),
    "no_keys": (1, 2, 40, 0, 128, 128, 0, False, 1.0),
    "d64_decode_step": (2, 3, 1, 777, 64, 64, 776, True, 1.0),
    "d64_chunk": (1, 3, 150, 1000, 64, 64, 850, True, 4.0),
    "d64_dv128_cross": (2, 2, 70, 403, 64, 128, 0, False, 1.0),
    "d64_dv128_causal": (1, 2, 257, 300, 64, 128, 43, True, 1.0),
}


def _random_general(n: int, seed: int):
    """Seeded random shapes beside the named ones (the same set on every run)."""
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        nk = int(rng.integers(1, 1101))
        causal = bool(rng.integers(0, 2))
        out["random_%02d" % i] = (int(rng.integers(1, 3)), int(rng.integers(1, 4)),
                                  int(rng.integers(1, 401)), nk, int(rng.choice([64, 128])),
                                  int(rng.choice([64, 128])),
                                  int(rng.integers(0, nk + 32)) if causal else 0, causal,
                                  float(rng.choice([1.0, 4.0])))
    return out


FP8_GENERAL.update(_random_general(6, 8808))


@pytest.mark.parametrize("name", sorted(FP8_GENERAL))
def test_fp8_general_shapes(name):
    B, H, Nq, Nk, d, dv, off, causal, mult = FP8_GENERAL[name]
    print("case fp8 general %s" % name, flush=True)
    ta = _ta()
    g = torch.Generator().manual_seed(500 + Nq + Nk)
    q = (torch.randn((B, H, Nq, d), generator=g) * mult).to(torch.bfloat16).contiguous()
    k = (torch.randn((B, H, Nk, d), generator=g) * mult).to(torch.bfloat16).contiguous()
    v = torch.randn((B, H, Nk, dv), generator=g).to(torch.bfloat16).contiguous()
    scale = 1 / np.sqrt(d)
    q8, qd = ta.attn_quantize_fp8(q.to(DEV))
    if Nk:
        k8, kd = ta.attn_quantize_fp8(k.to(DEV))
    else:
        k8 = torch.empty((B, H, 0, d), dtype=torch.uint8, device=DEV)
        kd = torch.ones((B, H), dtype=torch.float32, device=DEV)
    o, lse = ta.attn_fwd_fp8_ex(q8, k8, v.to(DEV), qd, kd, scale=scale, causal=causal,
                                query_offset=off)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    if Nk == 0:
        assert np.array_equal(o, np.zeros_like(o)) and np.all(lse == -np.inf)
        return
    rq8, rqd = quantize_per_head(_f64(q))
    rk8, rkd = quantize_per_head(_f64(k))
    assert np.array_equal(q8.cpu().numpy(), rq8) and np.array_equal(k8.cpu().numpy(), rk8)
    qf = e4m3_decode(rq8) * rqd[..., None, None].astype(np.float64)
    kf = e4m3_decode(rk8) * rkd[..., None, None].astype(np.float64)
    vf = _f64(v)
    errs_o, errs_l, bars = [], [], []
    for b in range(B):
        for h in range(H):
            ro, rl = attention_ref(qf[b, h], kf[b, h], vf[b, h], f32_scale(scale), causal,
                                   query_offset=off)
            vis = (np.arange(Nk)[None, :] <= (np.arange(Nq) + off)[:, None]) if causal else None
            bars.append(_lse_bar(qf[b, h], kf[b, h], scale, vis))
            errs_o.append(np.abs(o[b, h] - ro).ravel())
            errs_l.append(np.abs(lse[b, h] - rl))
    _check(np.concatenate(errs_o), np.concatenate(errs_l), np.concatenate(bars))


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_ex_square_equals_attn_fwd_fp8(d):
    """On a square problem with offset 0 the general instance gives the square
    instance's results bit for bit."""
    ta = _ta()
    print("case fp8 ex vs square d=%d" % d, flush=True)
    q, k, v = make_qkv(2, 2, 333, d, 95, 4.0)
    q8, qd = ta.attn_quantize_fp8(q.to(DEV))
    k8, kd = ta.attn_quantize_fp8(k.to(DEV))
    a = ta.attn_fwd_fp8(q8, k8, v.to(DEV), qd, kd, causal=True)
    b = ta.attn_fwd_fp8_ex(q8, k8, v.to(DEV), qd, kd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
