"""Pins for the oracle's bf16 round-to-nearest-even: agreement with torch's
float32 -> bfloat16 cast (an independent library routine) on random values
over the whole exponent range, exact midpoints, overflow and specials."""

import numpy as np
import pytest
import torch

from oracle import f32_to_bf16_rne, bf16_to_f32


def _torch_bits(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_random_values_match_torch():
    g = np.random.default_rng(1)
    bits = g.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(f32_to_bf16_rne(x), _torch_bits(x))


def test_exact_midpoints_round_to_even():
    g = np.random.default_rng(2)
    hi = g.integers(0, 0x7F7F, size=5000).astype(np.uint32)
    # exactly halfway between bf16 pattern `hi` and `hi + 1`
    mids = ((hi << 16) | 0x8000).view(np.float32)
    got = f32_to_bf16_rne(mids).astype(np.uint32)
    want = np.where(hi & 1, hi + 1, hi)
    assert np.array_equal(got, want)
    assert np.array_equal(got.astype(np.uint16), _torch_bits(mids))
    assert np.array_equal(f32_to_bf16_rne(-mids), _torch_bits(-mids))


def test_overflow_and_specials():
    x = np.array([3.3895314e38, 3.40e38, np.finfo(np.float32).max, np.inf, -np.inf,
                  0.0, -0.0, 1e-45, -1e-45, 1.1754942e-38], dtype=np.float32)
    assert np.array_equal(f32_to_bf16_rne(x), _torch_bits(x))
    nan = f32_to_bf16_rne(np.array([np.nan], dtype=np.float32))
    assert np.isnan(bf16_to_f32(nan))[0]


def test_bf16_to_f32_is_exact_upper_half():
    b = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(b)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(f[fin], ref[fin])
    assert np.array_equal(np.isnan(f), np.isnan(ref))


@pytest.mark.parametrize("v", [1.0, -2.5, 1e-20, 7.0e30])
def test_planted_truncation_is_caught(v):
    """Positive control: truncation instead of RNE disagrees with the library
    on values just above a midpoint."""
    x = np.array([v], dtype=np.float32)
    bits = x.view(np.uint32)
    above_mid = ((bits & 0xFFFF0000) | 0x8001).view(np.float32)
    trunc = (above_mid.view(np.uint32) >> 16).astype(np.uint16)
    assert not np.array_equal(trunc, _torch_bits(above_mid))
    assert np.array_equal(f32_to_bf16_rne(above_mid), _torch_bits(above_mid))
