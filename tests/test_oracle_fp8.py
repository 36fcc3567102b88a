"""CPU pins of the FP8 (E4M3, OCP fn variant) oracle: decoding of every code,
round-to-nearest-even encoding, and the per-head quantiser.

The independent reference is torch's float8_e4m3fn conversion (its own
implementation of the same published format)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode, quantize_per_head

ALL = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_every_code_matches_torch():
    ours, ref = e4m3_decode(ALL), _torch_decode(ALL)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_format_landmarks():
    v = e4m3_decode(ALL)
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    assert v[0x7E] == 448.0 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x01] == 2.0 ** -9                        # smallest subnormal
    assert v[0x08] == 2.0 ** -6                        # smallest normal
    assert v[0x38] == 1.0 and v[0x3C] == 1.5
    assert np.sum(np.isnan(v)) == 2


def test_encode_roundtrips_every_finite_code():
    fin = ALL[~np.isnan(e4m3_decode(ALL))]
    assert np.array_equal(e4m3_encode(e4m3_decode(fin)), fin)


def test_encode_ties_go_to_even_code():
    pos = np.arange(0x7E, dtype=np.uint8)                # adjacent pairs (c, c + 1)
    lo, hi = e4m3_decode(pos), e4m3_decode(pos + 1)
    mid = (lo + hi) / 2
    got = e4m3_encode(mid)
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(e4m3_encode(-mid), want | 0x80)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_encode_matches_torch_on_random_values(seed):
    rng = np.random.default_rng(seed)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.normal(0, 2.0 ** -8, 20000)]).astype(np.float32)
    assert np.array_equal(e4m3_encode(x.astype(np.float64)), _torch_encode(x))


def test_encode_matches_torch_on_midpoints():
    pos = np.arange(0x7E, dtype=np.uint8)
    mid = ((e4m3_decode(pos) + e4m3_decode(pos + 1)) / 2).astype(np.float32)
    assert np.array_equal(e4m3_encode(mid.astype(np.float64)), _torch_encode(mid))


def test_quantize_per_head():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 3, size=(2, 3, 50, 16)).astype(np.float32)
    x[1, 2] = 0.0                                        # an all-zero head
    codes, descale = quantize_per_head(x)
    assert codes.shape == x.shape and descale.shape == (2, 3)
    assert descale[1, 2] == 1.0 and np.all(codes[1, 2] & 0x7F == 0)
    back = e4m3_decode(codes) * descale[..., None, None]
    for b in range(2):
        for h in range(3):
            if b == 1 and h == 2:
                continue
            amax = np.abs(x[b, h]).max()
            assert np.isclose(descale[b, h], amax / 448, rtol=1e-7)
            i = np.unravel_index(np.argmax(np.abs(x[b, h])), x[b, h].shape)
            assert codes[b, h][i] & 0x7F == 0x7E         # the largest element maps to 448
            # 3 mantissa bits: relative error <= 2^-4 for normals, absolute <= 2^-10 * descale below
            err = np.abs(back[b, h] - x[b, h])
            assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x[b, h]), 2.0 ** -10 * descale[b, h]) + 1e-12)


def test_quantize_matches_torch_recipe():
    """The same float32 steps written with torch ops and torch's conversion."""
    rng = np.random.default_rng(6)
    x = rng.normal(0, 1.7, size=(4, 64, 32)).astype(np.float32)
    codes, descale = quantize_per_head(x)
    t = torch.from_numpy(x)
    amax = t.abs().amax(dim=(1, 2))
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    ref = (t * inv[:, None, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert np.array_equal(descale, (amax / 448.0).numpy())
