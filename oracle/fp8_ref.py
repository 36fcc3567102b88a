"""FP8 (E4M3, OCP "fn" variant) codes and per-head quantisation -- oracle side.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU leg
may use it; nothing is shared with the HIP path).

The pages name FP8 scores with online descaling as a lever of FlashAttention
v3 (page "Chapter 7 GPU Kernels: CUDA, HIP & Triton", sec. 7.6.2 and Figure
7.5) and ask that a low-precision product be compared with a reference on the
same quantised inputs (page "22. GPU Engineering: Correctness, Throughput, and
Attention", sec. 22.3).  The format itself is the OCP 8-bit E4M3 encoding:
1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
subnormal (value m/8 * 2^-6); there are no infinities; the only NaN pattern
is S.1111.111; the largest finite magnitude is 1.75 * 2^8 = 448.

Quantisation of one head (the reading taken here, since the pages fix no
recipe): amax = max |x| over the head; descale = amax / 448 (1 when amax = 0);
code = RNE_e4m3(clamp(x * (448 / amax), -448, 448)), each step one float32
operation in this order, so a float32 implementation reproduces every code.
"""
from __future__ import annotations

import numpy as np

__all__ = ["e4m3_decode", "e4m3_encode", "quantize_per_head", "E4M3_MAX"]

E4M3_MAX = 448.0


def _all_values() -> np.ndarray:
    """float64 value of every code 0..255 (NaN for the two NaN patterns)."""
    vals = np.empty(256)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_VALUES = _all_values()


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (exact)."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("expected uint8 codes")
    return _VALUES[c]


# Non-negative finite codes in increasing value order (0x00 .. 0x7E).
_POS = np.arange(0x7F, dtype=np.uint8)
_POS_VALS = _VALUES[_POS]


def e4m3_encode(x) -> np.ndarray:
    """Round float values to the nearest E4M3 code, ties to the even code
    (even mantissa), for |x| <= 448 (the caller clamps).  Zero keeps its sign."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values within +-448")
    a = np.abs(x)
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    exact = d_hi == 0
    pick_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS[hi] & 1) == 0))
    code = np.where(pick_hi, _POS[hi], _POS[lo]).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_per_head(x):
    """x: float array [..., rows, d] (one head per leading index), values as the
    device holds them (bf16 widened exactly).  Returns (codes uint8 of x's shape,
    descale float32 of shape x.shape[:-2]) with x ~= decode(codes) * descale."""
    x32 = np.asarray(x, dtype=np.float32)
    lead = x32.shape[:-2]
    flat = x32.reshape((-1,) + x32.shape[-2:])
    codes = np.empty(flat.shape, dtype=np.uint8)
    descale = np.empty(flat.shape[0], dtype=np.float32)
    for h in range(flat.shape[0]):
        amax = np.float32(np.max(np.abs(flat[h]))) if flat[h].size else np.float32(0)
        if amax == 0:
            inv = np.float32(1.0)
            descale[h] = np.float32(1.0)
        else:
            inv = np.float32(np.float32(E4M3_MAX) / amax)          # one float32 division
            descale[h] = np.float32(amax / np.float32(E4M3_MAX))
        scaled = np.clip(flat[h] * inv, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
        codes[h] = e4m3_encode(scaled.astype(np.float64))
    return codes.reshape(x32.shape), descale.reshape(lead)
