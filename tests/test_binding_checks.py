"""CPU tests of the Python binding's argument checks: every caller-supplied
output, workspace and input is checked for shape, dtype, contiguity and device
before the C entry point is called (a host tensor or a short buffer given as
an output would be written out of bounds by a kernel).

The stand-in ``Dev`` wraps a host tensor and reports itself as a device
tensor whose data pointer is NULL: a check that slipped through would reach
the C ABI, which rejects NULL pointers with a status (RuntimeError here),
never a launch.  So ``ValueError`` proves the wrapper stopped the call itself.
"""
from __future__ import annotations

import os

import pytest
import torch

import tiled_attention_09_amd as ta

pytestmark = pytest.mark.skipif(not os.path.exists(ta.library_path()),
                                reason="libtiledattn.so not built (run __graft_entry__.build())")

DEV = torch.device("cuda", 0)


class Dev:
    """A host tensor posing as a device tensor on cuda:0 (data pointer NULL)."""

    def __init__(self, shape, dtype, contiguous=True, device=DEV):
        self._t = torch.zeros(shape, dtype=dtype)
        self._contig = contiguous
        self.device = device
        self.is_cuda = device.type == "cuda"

    shape = property(lambda self: self._t.shape)
    dtype = property(lambda self: self._t.dtype)

    def dim(self):
        return self._t.dim()

    def is_contiguous(self):
        return self._contig

    def numel(self):
        return self._t.numel()

    def element_size(self):
        return self._t.element_size()

    def data_ptr(self):
        return 0


BF, F32, U8 = torch.bfloat16, torch.float32, torch.uint8
B, H, N, D = 1, 2, 128, 64


def qkv(n=N, d=D):
    return tuple(Dev((B, H, n, d), BF) for _ in range(3))


def bad_outputs(shape, dtype):
    """Wrong shape, wrong dtype, not contiguous, a real host tensor, another device."""
    short = (shape[:-1] + (shape[-1] - 1,)) if shape else (1,)
    other = torch.float64 if dtype != torch.float64 else torch.float32
    return [("shape", Dev(short, dtype)), ("dtype", Dev(shape, other)),
            ("contiguous", Dev(shape, dtype, contiguous=False)),
            ("host", torch.zeros(shape, dtype=dtype)),
            ("device", Dev(shape, dtype, device=torch.device("cuda", 1)))]


@pytest.mark.parametrize("kind,bad", bad_outputs((B, H, N, D), F32))
def test_attn_fwd_rejects_bad_out(kind, bad):
    q, k, v = qkv()
    with pytest.raises(ValueError):
        ta.attn_fwd(q, k, v, out=bad, lse=Dev((B, H, N), F32))


@pytest.mark.parametrize("kind,bad", bad_outputs((B, H, N), F32))
def test_attn_fwd_rejects_bad_lse(kind, bad):
    q, k, v = qkv()
    with pytest.raises(ValueError):
        ta.attn_fwd(q, k, v, out=Dev((B, H, N, D), F32), lse=bad)


def test_valid_stand_ins_reach_the_c_abi():
    """With valid metadata the wrapper calls the C entry point, which rejects the
    NULL data pointers by status: the stand-ins exercise the full wrapper path."""
    q, k, v = qkv()
    with pytest.raises(RuntimeError, match="invalid argument"):
        ta.attn_fwd(q, k, v, out=Dev((B, H, N, D), F32), lse=Dev((B, H, N), F32), stream=0)


@pytest.mark.parametrize("kind,bad", bad_outputs((B, H, N, D), F32))
def test_attn_fwd_dropout_rejects_bad_out(kind, bad):
    q, k, v = qkv()
    with pytest.raises(ValueError):
        ta.attn_fwd_dropout(q, k, v, 1, 26, out=bad, lse=Dev((B, H, N), F32))


@pytest.mark.parametrize("kind,bad", bad_outputs((B, H, 16, 128), F32))
def test_attn_fwd_ex_rejects_bad_out(kind, bad):
    q = Dev((B, H, 16, D), BF)
    k = Dev((B, H, 300, D), BF)
    v = Dev((B, H, 300, 128), BF)
    with pytest.raises(ValueError):
        ta.attn_fwd_ex(q, k, v, causal=True, query_offset=284, out=bad, lse=Dev((B, H, 16), F32))
    with pytest.raises(ValueError):
        ta.attn_fwd_split(q, k, v, causal=True, query_offset=284, out=bad,
                          lse=Dev((B, H, 16), F32), workspace=Dev((1 << 20,), U8))


def test_attn_fwd_split_rejects_bad_workspace():
    q = Dev((B, H, 16, D), BF)
    k = v = Dev((B, H, 300, D), BF)
    out, lse = Dev((B, H, 16, D), F32), Dev((B, H, 16), F32)
    for ws in (torch.zeros(1 << 20, dtype=U8), Dev((1 << 20,), U8, contiguous=False),
               Dev((1 << 20,), U8, device=torch.device("cuda", 1))):
        with pytest.raises(ValueError):
            ta.attn_fwd_split(q, k, v, out=out, lse=lse, workspace=ws)


def bwd_args():
    q, k, v = qkv()
    return q, k, v, Dev((B, H, N, D), F32), Dev((B, H, N), F32), Dev((B, H, N, D), BF)


@pytest.mark.parametrize("which", [0, 1, 2])
@pytest.mark.parametrize("kind,bad", bad_outputs((B, H, N, D), F32))
def test_attn_bwd_rejects_bad_grads(which, kind, bad):
    args = bwd_args()
    ws = Dev((ta.attn_bwd_workspace_size(B, H, N),), U8)
    grads = [Dev((B, H, N, D), F32) for _ in range(3)]
    grads[which] = bad
    with pytest.raises(ValueError):
        ta.attn_bwd(*args, workspace=ws, grads=grads)
    with pytest.raises(ValueError):
        ta.attn_bwd_dropout(*args, 1, 26, workspace=ws, grads=grads)
    with pytest.raises(ValueError):
        ta.attn_bwd_ex(*args, workspace=ws, grads=grads)


def test_attn_bwd_rejects_short_or_host_workspace():
    args = bwd_args()
    need = ta.attn_bwd_workspace_size(B, H, N)
    grads = [Dev((B, H, N, D), F32) for _ in range(3)]
    for ws in (Dev((need - 1,), U8), torch.zeros(need, dtype=U8)):
        with pytest.raises(ValueError):
            ta.attn_bwd(*args, workspace=ws, grads=grads)


@pytest.mark.parametrize("name", ["o", "lse", "do"])
def test_attn_bwd_rejects_host_inputs(name):
    q, k, v, o, lse, do = bwd_args()
    host = {"o": torch.zeros((B, H, N, D), dtype=F32), "lse": torch.zeros((B, H, N), dtype=F32),
            "do": torch.zeros((B, H, N, D), dtype=BF)}[name]
    kw = dict(o=o, lse=lse, do=do)
    kw[name] = host
    with pytest.raises(ValueError):
        ta.attn_bwd(q, k, v, kw["o"], kw["lse"], kw["do"])


def test_inputs_on_different_devices_are_rejected():
    q, k, v = qkv()
    k = Dev((B, H, N, D), BF, device=torch.device("cuda", 1))
    with pytest.raises(ValueError, match="must be on"):
        ta.attn_fwd(q, k, v, out=Dev((B, H, N, D), F32), lse=Dev((B, H, N), F32))


@pytest.mark.parametrize("kind,bad", bad_outputs((B, H, N, 128), U8))
def test_attn_quantize_fp8_rejects_bad_out(kind, bad):
    x = Dev((B, H, N, 128), BF)
    with pytest.raises(ValueError):
        ta.attn_quantize_fp8(x, out=bad, descale=Dev((B, H), F32))


@pytest.mark.parametrize("kind,bad", bad_outputs((B, H), F32))
def test_attn_quantize_fp8_rejects_bad_descale(kind, bad):
    x = Dev((B, H, N, 128), BF)
    with pytest.raises(ValueError):
        ta.attn_quantize_fp8(x, out=Dev((B, H, N, 128), U8), descale=bad)


@pytest.mark.parametrize("kind,bad", bad_outputs((B, H, N, 128), F32))
def test_attn_fwd_fp8_rejects_bad_out(kind, bad):
    q8, k8 = Dev((B, H, N, 128), U8), Dev((B, H, N, 128), U8)
    v = Dev((B, H, N, 128), BF)
    qd, kd = Dev((B, H), F32), Dev((B, H), F32)
    with pytest.raises(ValueError):
        ta.attn_fwd_fp8(q8, k8, v, qd, kd, out=bad, lse=Dev((B, H, N), F32))
    with pytest.raises(ValueError):
        ta.attn_fwd_fp8(q8, k8, v, qd, kd, out=Dev((B, H, N, 128), F32), lse=Dev((B, H, N + 1), F32))


def test_attn_fwd_fp8_rejects_host_descale():
    q8, k8 = Dev((B, H, N, 128), U8), Dev((B, H, N, 128), U8)
    v = Dev((B, H, N, 128), BF)
    with pytest.raises(ValueError):
        ta.attn_fwd_fp8(q8, k8, v, torch.ones((B, H)), Dev((B, H), F32),
                        out=Dev((B, H, N, 128), F32), lse=Dev((B, H, N), F32))
