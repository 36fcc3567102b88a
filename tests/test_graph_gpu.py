"""The entry points under HIP graph capture: each call only enqueues kernels
on the given stream (no allocation, no memset node, no host synchronisation),
so a captured sequence replays to the same bits as the eager calls.  Every
replay is checked, with unrelated eager work and synchronisations between
replays, and the inputs are changed in place between replays to show the graph
reads them at replay time."""
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


def test_forward_backward_fp8_dropout_replay_like_eager():
    print("case graph capture B=2 H=4 N=700 d=128 causal", flush=True)
    ta = _ta()
    B, H, N, d = 2, 4, 700, 128
    q, k, v = (x.to(DEV) for x in make_qkv(B, H, N, d, 61))
    g = make_dout(B, H, N, d, 61).to(DEV)
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    od = torch.empty_like(o)
    lsed = torch.empty_like(lse)
    o8 = torch.empty_like(o)
    lse8 = torch.empty_like(lse)
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=DEV)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=DEV)
    qs = torch.empty((B, H), dtype=torch.float32, device=DEV)
    ks = torch.empty((B, H), dtype=torch.float32, device=DEV)
    ws = torch.empty(ta.attn_bwd_workspace_size(B, H, N), dtype=torch.uint8, device=DEV)
    grads = tuple(torch.empty_like(o) for _ in range(3))

    def run(stream):
        sc = stream.cuda_stream
        ta.attn_fwd(q, k, v, causal=True, out=o, lse=lse, stream=sc)
        ta.attn_bwd(q, k, v, o, lse, g, causal=True, workspace=ws, grads=grads, stream=sc)
        ta.attn_fwd_dropout(q, k, v, 5, 40, causal=True, out=od, lse=lsed, stream=sc)
        ta.attn_quantize_fp8(q, out=q8, descale=qs, stream=sc)
        ta.attn_quantize_fp8(k, out=k8, descale=ks, stream=sc)
        ta.attn_fwd_fp8(q8, k8, v, qs, ks, causal=True, out=o8, lse=lse8, stream=sc)

    outs = (o, lse, od, lsed, o8, lse8, q8, k8, qs, ks) + grads
    side = torch.cuda.Stream(DEV)
    # eager reference
    with torch.cuda.stream(side):
        run(side)
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    for t in outs:
        t.zero_()
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run(side)
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), "replay %d differs from the eager result" % rep
        # unrelated eager work and a clobber of the outputs between replays
        junk = torch.randn(1 << 20, device=DEV).sum()
        for t in outs:
            t.fill_(7)
        torch.cuda.synchronize()
        assert torch.isfinite(junk)

    # the graph reads its inputs at replay time
    q.mul_(-1)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    o_new = o.clone()
    with torch.cuda.stream(side):
        ta.attn_fwd(q, k, v, causal=True, out=o, lse=lse, stream=side.cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o_new, o)
    assert not torch.equal(o_new, want[0])
