"""GPU parity of the general-shape forward (attn_fwd_ex) against the float64 oracle.

Shapes from the lab's conventions (page "22. GPU Engineering: Correctness,
Throughput, and Attention", sec. 22.7): Nq queries at absolute positions
query_offset + i attending Nk keys (decoding steps, chunks of queries, more
queries than keys), value width dv != d, and the policy for rows that see no
key.  Same bar as the square forward: max |dO| <= 1e-2, mean |dO| <= 1e-3,
max |dLSE| <= 1e-3; every row compared.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention_ref, bf16_bits_to_f64, f32_scale
from tiled_attention_09_amd.synth import bf16_bits

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3


def _ta():
    import tiled_attention_09_amd as ta
    ta.load_library()
    return ta


def _inputs(B, H, Nq, Nk, d, dv, seed, qk_mult=1.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g) * qk_mult
    k = torch.randn((B, H, Nk, d), generator=g) * qk_mult
    v = torch.randn((B, H, Nk, dv), generator=g)
    return tuple(x.to(torch.bfloat16).contiguous() for x in (q, k, v))


def _f64(t):
    return bf16_bits_to_f64(bf16_bits(t))


def _oracle(q, k, v, scale, causal, off):
    B, H, Nq = q.shape[:3]
    dv = v.shape[3]
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    ro = np.zeros((B, H, Nq, dv))
    rl = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            ro[b, h], rl[b, h] = attention_ref(qd[b, h], kd[b, h], vd[b, h], f32_scale(scale), causal,
                                               query_offset=off)
    return ro, rl


CASES = {  # name: (B, H, Nq, Nk, d, dv, offset, causal, qk_mult, scale)
    "decode_first": (2, 4, 1, 1, 128, 128, 0, True, 1.0, None),
    "decode_77": (2, 4, 1, 77, 128, 128, 76, True, 1.0, None),
    "decode_1000_dv64": (2, 4, 1, 1000, 128, 64, 999, True, 1.0, None),
    "decode_4096_d64_dv128": (1, 8, 1, 4096, 64, 128, 4095, True, 1.0, None),
    "decode_32768": (1, 16, 1, 32768, 128, 128, 32767, True, 1.0, None),
    "chunk_100_of_1000": (1, 4, 100, 1000, 128, 128, 900, True, 1.0, None),
    "chunk_257_of_1024_d64": (2, 2, 257, 1024, 64, 64, 767, True, 1.0, None),
    "more_queries_noncausal": (1, 2, 300, 50, 128, 128, 0, False, 1.0, None),
    "more_queries_causal": (1, 2, 300, 100, 64, 64, 0, True, 1.0, None),
    "offset_past_keys": (1, 2, 64, 100, 128, 64, 500, True, 1.0, None),
    "square_d64_dv128": (2, 3, 333, 333, 64, 128, 0, True, 1.0, None),
    "square_d128_dv64": (2, 3, 333, 333, 128, 64, 0, False, 1.0, None),
    "chunk_large_logits": (1, 2, 200, 700, 128, 128, 500, True, 4.0, None),
    "chunk_negative_scale": (1, 2, 130, 390, 64, 128, 260, True, 4.0, -0.125),
    # 8 heads, 3 query tiles each: causal tiles taken longest first across heads
    "chunk_300_of_1200_8heads": (2, 4, 300, 1200, 128, 128, 900, True, 1.0, None),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_general_shape(name):
    B, H, Nq, Nk, d, dv, off, causal, mult, scale = CASES[name]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    print("case %s: B=%d H=%d Nq=%d Nk=%d d=%d dv=%d offset=%d causal=%d" % (
        name, B, H, Nq, Nk, d, dv, off, causal), flush=True)
    q, k, v = _inputs(B, H, Nq, Nk, d, dv, 500 + Nq + Nk + d + dv, mult)
    o, lse = _ta().attn_fwd_ex(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal,
                               query_offset=off)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    ro, rl = _oracle(q, k, v, scale, causal, off)
    do, dl = np.abs(o - ro), np.abs(lse - rl)
    msg = "%s: max|dO| %.3e mean|dO| %.3e max|dLSE| %.3e" % (name, do.max(), do.mean(), dl.max())
    print(msg, flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), msg
    assert do.max() <= O_MAX and do.mean() <= O_MEAN and dl.max() <= LSE_MAX, msg


def test_no_keys_policy():
    """Nk = 0: every row sees no key -> O = 0 and LSE = -inf exactly (lab policy)."""
    q, k, v = _inputs(1, 2, 70, 0, 128, 64, 9)
    o, lse = _ta().attn_fwd_ex(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, query_offset=3)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 70, 64)
    assert torch.all(o.cpu() == 0)
    assert torch.all(torch.isneginf(lse.cpu()))


def test_square_call_is_the_general_one():
    """attn_fwd(N) and attn_fwd_ex(N, N, d, d, offset 0) give identical bits."""
    ta = _ta()
    q, k, v = (t.to(DEV) for t in _inputs(2, 3, 1003, 1003, 64, 64, 11))
    for causal in (False, True):
        a = ta.attn_fwd(q, k, v, causal=causal)
        b = ta.attn_fwd_ex(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_query_chunk_equals_rows_of_full_problem():
    """The last 300 rows of a causal N = 2000 problem, computed as a chunk of
    queries at offset 1700, agree with the full problem's rows."""
    ta = _ta()
    q, k, v = (t.to(DEV) for t in _inputs(1, 4, 2000, 2000, 128, 128, 12))
    full_o, full_l = ta.attn_fwd(q, k, v, causal=True)
    o, l = ta.attn_fwd_ex(q[:, :, 1700:].contiguous(), k, v, causal=True, query_offset=1700)
    torch.cuda.synchronize()
    assert (o - full_o[:, :, 1700:]).abs().max().item() <= 1e-6
    assert (l - full_l[:, :, 1700:]).abs().max().item() <= 1e-6
