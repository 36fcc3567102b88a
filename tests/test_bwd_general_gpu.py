"""GPU parity of the general-shape backward (attn_bwd_ex) against the float64
oracle: Nq queries at positions query_offset + i and Nk keys, value width
dv != d (page "22. GPU Engineering: Correctness, Throughput, and Attention",
sec. 22.7: the lab's decoding-style subproblems; sec. 22.5 for the gradients).
Full path: the HIP general forward's O and LSE feed the HIP backward; the
oracle computes the gradients from its exact probabilities.  Bars as for the
square backward, per gradient X: max |X - X_ref| <= 2^-6 max |X_ref| + 1e-5,
mean |X - X_ref| <= 2^-8 mean |X_ref| + 1e-6; every row compared.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention_bwd_ref, bf16_bits_to_f64, f32_scale
from tiled_attention_09_amd.synth import bf16_bits

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MAX_REL, MEAN_REL = 2.0 ** -6, 2.0 ** -8


def _ta():
    import tiled_attention_09_amd as ta
    ta.load_library()
    return ta


def _f64(t):
    return bf16_bits_to_f64(bf16_bits(t))


def _inputs(B, H, Nq, Nk, d, dv, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g) * mult
    k = torch.randn((B, H, Nk, d), generator=g) * mult
    v = torch.randn((B, H, Nk, dv), generator=g)
    do = torch.randn((B, H, Nq, dv), generator=g)
    return tuple(x.to(torch.bfloat16).contiguous() for x in (q, k, v, do))


def _check(name, got, ref):
    err = np.abs(got - ref)
    mx = np.abs(ref).max() if ref.size else 0.0
    mean = np.abs(ref).mean() if ref.size else 0.0
    msg = "%s max %.2e (of %.2e) mean %.2e (of %.2e)" % (
        name, err.max() if err.size else 0, mx, err.mean() if err.size else 0, mean)
    print("  " + msg, flush=True)
    assert np.all(np.isfinite(got)), msg
    if err.size:
        assert err.max() <= MAX_REL * mx + 1e-5 and err.mean() <= MEAN_REL * mean + 1e-6, msg


CASES = {  # name: (B, H, Nq, Nk, d, dv, offset, causal, mult, scale)
    "decode_77": (2, 3, 1, 77, 128, 128, 76, True, 1.0, None),
    "decode_1000_dv64": (1, 4, 1, 1000, 128, 64, 999, True, 1.0, None),
    "decode_513_d64_dv128": (1, 2, 1, 513, 64, 128, 512, True, 1.0, None),
    "chunk_100_of_1000": (1, 4, 100, 1000, 128, 128, 900, True, 1.0, None),
    "chunk_257_of_1024_d64": (2, 2, 257, 1024, 64, 64, 767, True, 1.0, None),
    "more_queries_noncausal": (1, 2, 300, 50, 128, 128, 0, False, 1.0, None),
    "more_queries_causal": (1, 2, 300, 100, 64, 64, 0, True, 1.0, None),
    "offset_past_keys": (1, 2, 64, 100, 128, 64, 500, True, 1.0, None),
    "square_d64_dv128": (2, 3, 333, 333, 64, 128, 0, True, 1.0, None),
    "square_d128_dv64": (2, 3, 333, 333, 128, 64, 0, False, 1.0, None),
    "chunk_large_logits": (1, 2, 200, 700, 128, 128, 500, True, 4.0, None),
    "chunk_negative_scale": (1, 2, 130, 390, 64, 128, 260, True, 4.0, -0.125),
    "ragged_noncausal_dv64": (2, 2, 129, 191, 128, 64, 0, False, 1.0, None),
    # 8 heads with few query and key tiles: causal tiles taken longest first across heads
    "chunk_300_of_1200_8heads": (2, 4, 300, 1200, 128, 128, 900, True, 1.0, None),
    "chunk_200_of_600_8heads_d64": (2, 4, 200, 600, 64, 64, 400, True, 1.0, None),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_general_backward(name):
    B, H, Nq, Nk, d, dv, off, causal, mult, scale = CASES[name]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    print("case bwd_ex %s: B=%d H=%d Nq=%d Nk=%d d=%d dv=%d offset=%d causal=%d" % (
        name, B, H, Nq, Nk, d, dv, off, causal), flush=True)
    ta = _ta()
    q, k, v, do = _inputs(B, H, Nq, Nk, d, dv, 700 + Nq + Nk + d + dv, mult)
    qd, kd, vd, gd = (x.to(DEV) for x in (q, k, v, do))
    o, lse = ta.attn_fwd_ex(qd, kd, vd, scale=scale, causal=causal, query_offset=off)
    dq, dk, dvg = ta.attn_bwd_ex(qd, kd, vd, o, lse, gd, scale=scale, causal=causal,
                                 query_offset=off)
    torch.cuda.synchronize()
    dq, dk, dvg = (x.cpu().double().numpy() for x in (dq, dk, dvg))
    rq, rk, rv = (np.zeros(x.shape) for x in (dq, dk, dvg))
    for b in range(B):
        for h in range(H):
            rq[b, h], rk[b, h], rv[b, h] = attention_bwd_ref(
                _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(do[b, h]), f32_scale(scale),
                causal, off)
    _check("dQ", dq, rq)
    _check("dK", dk, rk)
    _check("dV", dvg, rv)


def test_empty_query_or_key_sets():
    """Nq = 0: dK = dV = 0 for every key; Nk = 0: dQ = 0 for every query."""
    ta = _ta()
    q, k, v, do = (x.to(DEV) for x in _inputs(1, 2, 0, 70, 128, 64, 5))
    o = torch.empty((1, 2, 0, 64), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device=DEV)
    grads = (torch.full((1, 2, 0, 128), 7.0, device=DEV), torch.full((1, 2, 70, 128), 7.0, device=DEV),
             torch.full((1, 2, 70, 64), 7.0, device=DEV))
    dq, dk, dv = ta.attn_bwd_ex(q, k, v, o, lse, do, causal=True, query_offset=3, grads=grads)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)

    q, k, v, do = (x.to(DEV) for x in _inputs(1, 2, 40, 0, 64, 128, 6))
    o, lse = ta.attn_fwd_ex(q, k, v, causal=True, query_offset=9)
    grads = (torch.full((1, 2, 40, 64), 7.0, device=DEV), torch.full((1, 2, 0, 64), 7.0, device=DEV),
             torch.full((1, 2, 0, 128), 7.0, device=DEV))
    dq, dk, dv = ta.attn_bwd_ex(q, k, v, o, lse, do, causal=True, query_offset=9, grads=grads)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


def test_square_backward_through_the_general_entry():
    """attn_bwd_ex with Nq = Nk, offset 0, dv = d agrees with attn_bwd (a
    different kernel instance: equal up to fp32 rounding order)."""
    ta = _ta()
    q, k, v, do = (x.to(DEV) for x in _inputs(2, 2, 300, 300, 128, 128, 8))
    for causal in (False, True):
        o, lse = ta.attn_fwd(q, k, v, causal=causal)
        a = ta.attn_bwd(q, k, v, o, lse, do, causal=causal)
        b = ta.attn_bwd_ex(q, k, v, o, lse, do, causal=causal)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert (x - y).abs().max().item() <= 1e-5 * max(1.0, x.abs().max().item())
