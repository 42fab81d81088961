"""Pins for the oracle's bfloat16 conversions (CPU only)."""
import numpy as np
import pytest
import torch

from oracle.numerics import bf16_to_f32, f32_to_bf16


def _f(bits32):
    return np.array([bits32], dtype=np.uint32).view(np.float32)


def test_upcast_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x0000, 0x8000], dtype=np.uint16)
    got = bf16_to_f32(bits)
    assert got[0] == 1.0 and got[1] == -2.0
    assert np.isposinf(got[2]) and np.isneginf(got[3])
    assert got[4] == np.float32(2.0 ** -133)       # smallest bf16 subnormal
    assert got[5] == 0.0 and np.signbit(got[6])


@pytest.mark.parametrize("value,expect", [
    (1.0, 0x3F80),
    (1.0 + 2 ** -8, 0x3F80),           # exact tie -> even (down)
    (1.0 + 3 * 2 ** -8, 0x3F82),       # exact tie -> even (up)
    (1.0 + 2 ** -8 + 2 ** -20, 0x3F81),  # just above the tie -> up
    (1.0 + 2 ** -8 - 2 ** -20, 0x3F80),  # just below the tie -> down
    (-(1.0 + 3 * 2 ** -8), 0xBF82),
    (3.0e38, 0x7F62),
])
def test_round_to_nearest_even_closed_forms(value, expect):
    assert int(f32_to_bf16(np.array([value], dtype=np.float32))[0]) == expect


def test_overflow_and_nan():
    assert int(f32_to_bf16(_f(0x7F7FFFFF))[0]) == 0x7F80   # rounds up to +inf
    out = f32_to_bf16(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.isnan(bf16_to_f32(out)).all()


def test_matches_torch_conversion():
    """Special case reducing to a library routine: torch's float32 ->
    bfloat16 cast is round-to-nearest-even too."""
    g = torch.Generator().manual_seed(0)
    x = torch.cat([torch.randn(200000, generator=g) * 10.0 ** torch.randint(-30, 30, (200000,), generator=g),
                   torch.tensor([0.0, -0.0, 1e-40, -3e-39, float("inf"), float("-inf")])])
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f32_to_bf16(x.numpy())
    assert np.array_equal(got, ref)


def test_round_trip_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(bits)
    ok = ~np.isnan(f)
    assert np.array_equal(f32_to_bf16(f)[ok], bits[ok])
