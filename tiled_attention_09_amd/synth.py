"""Seeded synthetic inputs for attention forward, shared by tests and benchmark.

This module only draws random numbers and picks rows; it contains none of the
attention arithmetic, so both the oracle side and the HIP side may consume its
output without sharing any of the method.

Recipe (every workload): a CPU ``torch.Generator`` seeded with the workload's
seed draws standard-normal float32 tensors of shape [B, H, N, d] in the order
Q, K, V; Q and K are multiplied by ``qk_mult`` (a power of two, so the
multiplication is exact); all three are rounded to bfloat16 with
round-to-nearest-even.  Sampled query rows use a second generator seeded with
``seed + 100``.  The output gradient G of the backward is a standard-normal
[B, H, N, d] tensor from a generator seeded with ``seed + 200``, rounded to
bfloat16 the same way.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "make_dout", "sample_rows", "bf16_bits",
           "headline"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    qk_mult: float = 1.0
    full_oracle: bool = True     # False: parity on sampled rows per head

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Algorithmic flops: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def bwd_flops(self) -> float:
        """Algorithmic backward flops: five products of 2*N^2*d each (dV, dP, dQ,
        dK and the recomputed scores), 10*B*H*N^2*d, halved when causal."""
        return 2.5 * self.flops

    @property
    def alg_bytes(self) -> int:
        """Read Q, K, V (bf16) once; write O (fp32) and LSE (fp32) once."""
        n = self.B * self.H * self.N
        return 3 * n * self.d * 2 + n * self.d * 4 + n * 4

    def describe(self) -> str:
        mult = "" if self.qk_mult == 1.0 else ", Q,K x%g" % self.qk_mult
        return "B=%d,H=%d,N=%d,d=%d,%s%s" % (self.B, self.H, self.N, self.d,
                                            "causal" if self.causal else "non-causal", mult)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 128, 64, False, 1),
    "ragged": Workload("ragged", 4, 8, 1003, 64, False, 2),
    "mid_causal": Workload("mid_causal", 8, 16, 2048, 128, True, 3),
    "headline": Workload("headline", 2, 32, 8192, 128, True, 4, qk_mult=4.0, full_oracle=False),
    "long": Workload("long", 1, 16, 32768, 128, True, 5, full_oracle=False),
}


def headline() -> Workload:
    return WORKLOADS["headline"]


def make_qkv(B: int, H: int, N: int, d: int, seed: int, qk_mult: float = 1.0):
    """Return (q, k, v) as contiguous CPU bfloat16 tensors of shape [B, H, N, d]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if qk_mult != 1.0:
        q.mul_(qk_mult)
        k.mul_(qk_mult)
    return (q.to(torch.bfloat16).contiguous(), k.to(torch.bfloat16).contiguous(),
            v.to(torch.bfloat16).contiguous())


def make_workload(w: Workload):
    return make_qkv(w.B, w.H, w.N, w.d, w.seed, w.qk_mult)


def make_dout(B: int, H: int, N: int, d: int, seed: int) -> torch.Tensor:
    """The output gradient G: contiguous CPU bfloat16 [B, H, N, d]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 200)
    return torch.randn((B, H, N, d), generator=g, dtype=torch.float32).to(torch.bfloat16).contiguous()


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Sorted unique query rows: fixed tile-edge rows plus seeded uniform fill."""
    fixed = [r for r in (0, 1, 63, 64, 127, 128, 129, N - 2, N - 1) if 0 <= r < N]
    chosen = set(fixed)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    target = min(count, N)
    while len(chosen) < target:
        draw = torch.randint(0, N, (target,), generator=g).tolist()
        for r in draw:
            if len(chosen) >= target:
                break
            chosen.add(int(r))
    return np.array(sorted(chosen), dtype=np.int64)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a CPU bfloat16 tensor (no arithmetic)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
