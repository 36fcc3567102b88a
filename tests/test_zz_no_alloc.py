"""GPU test of attn_bwd_noalloc, the backward that allocates nothing (its row
statistics live in the library's fixed device scratch): through the C ABI, its
gradients equal attn_bwd's (workspace from the caller) bit for bit, on two
calls in a row, the second with a smaller problem (the scratch keeps the first
call's contents, which must not leak into the second).  Outputs start as NaN so
every element must be written."""
from __future__ import annotations

import pytest
import torch

from tiled_attention_09_amd.synth import make_dout, make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _ta():
    import tiled_attention_09_amd as ta
    ta.load_library()
    return ta


def _one_call(ta, B, H, N, d, causal, seed):
    print("case noalloc B=%d H=%d N=%d d=%d causal=%d" % (B, H, N, d, causal), flush=True)
    q, k, v = (x.to(DEV) for x in make_qkv(B, H, N, d, seed))
    g = make_dout(B, H, N, d, seed).to(DEV)
    scale = d ** -0.5
    o, lse = ta.attn_fwd(q, k, v, scale, causal)
    ref = ta.attn_bwd(q, k, v, o, lse, g, scale, causal)
    got = tuple(torch.full((B, H, N, d), float("nan"), device=DEV) for _ in range(3))
    stream = torch.cuda.current_stream(DEV).cuda_stream
    st = ta.attn_bwd_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), g.data_ptr(), got[0].data_ptr(),
                                 got[1].data_ptr(), got[2].data_ptr(), B, H, N, d, scale,
                                 int(causal), stream)
    assert st == ta.TA_OK, ta.attn_status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(a).all(), name
        assert torch.equal(a, b), "%s differs from attn_bwd: max %.3e" % (
            name, (a - b).abs().max().item())


def test_noalloc_equals_attn_bwd_on_two_calls():
    ta = _ta()
    _one_call(ta, 2, 8, 1000, 128, True, 31)     # 16 000 rows of scratch statistics
    _one_call(ta, 1, 3, 257, 64, False, 32)      # then a smaller problem


def test_noalloc_python_wrapper():
    ta = _ta()
    q, k, v = (x.to(DEV) for x in make_qkv(1, 2, 300, 64, 33))
    g = make_dout(1, 2, 300, 64, 33).to(DEV)
    o, lse = ta.attn_fwd(q, k, v, causal=True)
    ref = ta.attn_bwd(q, k, v, o, lse, g, causal=True)
    got = ta.attn_bwd_noalloc(q, k, v, o, lse, g, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
