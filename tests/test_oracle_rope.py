"""Pins for the oracle's 3D rotary embedding (CPU only).

The pages fix that K is rotated before publishing ("Wave Forcing", §4.2) and
the configurations fix the sub-band split and theta; the rotation itself is
the textbook one.  These tests pin it with closed-form angles (cos/sin of
1, 2, 3 and 0.5 rad), identity at position 0, norm preservation, the
relative-position property per axis, and axis separation.
"""
import math

import numpy as np
import pytest

from oracle.numerics import bf16_to_f32, f32_to_bf16
from oracle.rope import apply_rope, axis_of_pair, rotate_f32, rotate_f64


def _unit(D, j):
    x = np.zeros((1, 1, D), dtype=np.float32)
    x[0, 0, j] = 1.0
    return x


# (split, element pair p, position (t, h, w), angle in rad)
# - 24/20/20, w axis, i = 5: omega = 10000^(-10/20) = 0.01, pos 100 -> 1 rad
# - 44/42/42, t axis, i = 11: omega = 10000^(-22/44) = 0.01, pos 50 -> 0.5 rad
# - 44/42/42, h axis, i = 0: omega = 1, pos 2 -> 2 rad
# - 44/42/42, t axis, i = 0: omega = 1, pos 3 -> 3 rad
# - 24/20/20, h axis, i = 5: omega = 0.01, pos 300 -> 3 rad
CASES = [
    ((24, 20, 20), 22 + 5, (0, 0, 100), 1.0),
    ((44, 42, 42), 11, (50, 0, 0), 0.5),
    ((44, 42, 42), 22, (0, 2, 0), 2.0),
    ((44, 42, 42), 0, (3, 0, 0), 3.0),
    ((24, 20, 20), 12 + 5, (0, 300, 0), 3.0),
]
COS = {1.0: 0.5403023058681398, 0.5: 0.8775825618903728,
       2.0: -0.4161468365471424, 3.0: -0.9899924966004454}
SIN = {1.0: 0.8414709848078965, 0.5: 0.479425538604203,
       2.0: 0.9092974268256817, 3.0: 0.1411200080598672}


@pytest.mark.parametrize("split,p,pos,angle", CASES)
def test_closed_form_rotation(split, p, pos, angle):
    D = sum(split)
    P = np.array([pos], dtype=np.int32)
    c, s = np.float32(COS[angle]), np.float32(SIN[angle])
    y = rotate_f32(_unit(D, 2 * p), P, split, 10000.0)[0, 0]
    expect = np.zeros(D, dtype=np.float32)
    expect[2 * p], expect[2 * p + 1] = c, s          # e0 -> (cos, sin)
    assert np.array_equal(y, expect)
    y = rotate_f32(_unit(D, 2 * p + 1), P, split, 10000.0)[0, 0]
    expect[:] = 0
    expect[2 * p], expect[2 * p + 1] = -s, c         # e1 -> (-sin, cos)
    assert np.array_equal(y, expect)


def test_axis_of_pair_bands():
    split = (44, 42, 42)
    axes = [axis_of_pair(p, split) for p in range(64)]
    assert axes[0] == (0, 0) and axes[21] == (0, 21)
    assert axes[22] == (1, 0) and axes[42] == (1, 20)
    assert axes[43] == (2, 0) and axes[63] == (2, 20)


@pytest.mark.parametrize("split", [(24, 20, 20), (44, 42, 42)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_identity_at_position_zero(split, dtype):
    rng = np.random.default_rng(0)
    D = sum(split)
    x = rng.standard_normal((50, 3, D)).astype(np.float32)
    if dtype == "bf16":
        x = bf16_to_f32(f32_to_bf16(x))
    out = apply_rope(x, np.zeros((50, 3), np.int32), split, 10000.0, dtype)
    ref = f32_to_bf16(x) if dtype == "bf16" else x
    assert np.array_equal(out, ref)


def test_axis_separation():
    """A position on one axis rotates exactly that axis's sub-band."""
    split = (44, 42, 42)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 2, 128)).astype(np.float32)
    bands = [(0, 44), (44, 86), (86, 128)]
    for a in range(3):
        pos = np.zeros((4, 3), np.int32)
        pos[:, a] = [1, 5, 17, 29]
        y = rotate_f32(x, pos, split, 10000.0)
        for b, (lo, hi) in enumerate(bands):
            same = np.array_equal(y[..., lo:hi], x[..., lo:hi])
            assert same == (a != b)


def test_norm_preserved_per_pair():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 2, 128))
    pos = rng.integers(0, 60, size=(64, 3)).astype(np.int32)
    y = rotate_f64(x, pos, (44, 42, 42), 10000.0)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_relative_position_property(axis):
    """<R(p+d) q, R(p'+d) k> = <R(p) q, R(p') k>: scores depend on the
    position difference along each axis only."""
    rng = np.random.default_rng(3 + axis)
    split = (44, 42, 42)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    for p, pp, d in [(0, 7, 5), (3, 3, 40), (11, 2, 19)]:
        a = np.zeros((1, 3), np.int32)
        b = np.zeros((1, 3), np.int32)
        a[0, axis], b[0, axis] = p, pp
        base = float(np.sum(rotate_f64(q, a, split, 1e4) * rotate_f64(k, b, split, 1e4)))
        a[0, axis] += d
        b[0, axis] += d
        moved = float(np.sum(rotate_f64(q, a, split, 1e4) * rotate_f64(k, b, split, 1e4)))
        assert math.isclose(base, moved, rel_tol=1e-11, abs_tol=1e-11)


def test_float32_path_tracks_float64():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((200, 2, 128)).astype(np.float32)
    pos = rng.integers(0, 80, size=(200, 3)).astype(np.int32)
    y32 = rotate_f32(x, pos, (44, 42, 42), 1e4).astype(np.float64)
    y64 = rotate_f64(x.astype(np.float64), pos, (44, 42, 42), 1e4)
    np.testing.assert_allclose(y32, y64, rtol=0, atol=3e-6)


# ---- the rounding rule of the rotation (R9) --------------------------------
# The precision reading of the publish (K rotated before publishing, "Wave
# Forcing", §4.2): cos and sin rounded to float32, then
#   y0 = f32(f32(x0*c) - f32(x1*s)),   y1 = f32(f32(x0*s) + f32(x1*c)),
# each product and the sum rounded on its own (no fused multiply-add), then
# round-to-nearest-even to the storage type.  Hand-worked cases at the 1 rad
# angle of the closed-form table (split 24/20/20, pair 27, w position 100;
# c = f32(cos 1) = 0x3f0a5140, s = f32(sin 1) = 0x3f576aa4), with inputs
# chosen so that the per-operation result, the single-rounding result
# f32(x0*c - x1*s) and the fused result f32(x0*c - f32(x1*s)) all differ.
# Each row: output (0: y0, 1: y1), x0 bits, x1 bits, then the per-operation
# float32 bits (the reading), the single-rounding and fused float32 bits, and
# the bfloat16 bits of the reading and of the single rounding.  The float32
# values were worked out with exact rational arithmetic and explicit
# round-to-nearest-even; test_rounding_cases_are_exact re-derives them.
R9_CASES = [
    # y0 = x0*c - x1*s
    (0, 0xbf887961, 0xbf2d7ae9, 0xbbbf8000, 0xbbbf7ff5, 0xbbbf7fd0, 0xbbc0, 0xbbbf),
    (0, 0x3f116cee, 0x3eb9bbfd, 0x3adb8000, 0x3adb7fef, 0x3adb803d, 0x3adc, 0x3adb),
    # y1 = x0*s + x1*c
    (1, 0x3f241f3e, 0xbf7e7582, 0x3b1e8000, 0x3b1e8046, 0x3b1e8026, 0x3b1e, 0x3b1f),
    (1, 0xbf2db598, 0x3f86c2a0, 0xbb0c8000, 0xbb0c8017, 0xbb0c8021, 0xbb0c, 0xbb0d),
    (1, 0xbf9c7a40, 0x3ff3727d, 0xba8b8000, 0xba8b7c93, 0xba8b7e73, 0xba8c, 0xba8b),
]
R9_C, R9_S = 0x3f0a5140, 0x3f576aa4


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def _bits(x):
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def _rne(fr, mant_bits):
    """Round a nonzero rational to `mant_bits` significand bits, ties to even
    (normal range)."""
    from fractions import Fraction
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    q = a / ulp
    n, rem = divmod(q.numerator, q.denominator)
    rem = Fraction(rem, q.denominator)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def test_rounding_factors_of_the_case_angle():
    # the 1 rad factors of the case table, rounded from double precision
    assert _bits(np.float32(COS[1.0])) == R9_C and _bits(np.float32(SIN[1.0])) == R9_S
    from oracle.rope import pair_factors
    c, s = pair_factors(np.array([[0, 0, 100]]), (24, 20, 20), 10000.0)
    assert _bits(c[0, 27]) == R9_C and _bits(s[0, 27]) == R9_S


@pytest.mark.parametrize("case", R9_CASES)
def test_rounding_cases_are_exact(case):
    from fractions import Fraction as Fr
    out, bx0, bx1, per_op, single, fused, bf_per_op, bf_single = case
    x0, x1 = Fr(float(_f32(bx0))), Fr(float(_f32(bx1)))
    c, s = Fr(float(_f32(R9_C))), Fr(float(_f32(R9_S)))
    if out == 0:
        a, b, sign = x0 * c, x1 * s, -1
    else:
        a, b, sign = x0 * s, x1 * c, 1
    r = _rne(_rne(a, 24) + sign * _rne(b, 24), 24)
    assert _bits(float(r)) == per_op
    assert _bits(float(_rne(a + sign * b, 24))) == single
    assert _bits(float(_rne(a + sign * _rne(b, 24), 24))) == fused
    assert _bits(float(_rne(r, 8))) >> 16 == bf_per_op
    assert _bits(float(_rne(_rne(a + sign * b, 24), 8))) >> 16 == bf_single
    # the three readings are distinguishable on these inputs
    assert len({per_op, single, fused}) == 3 and bf_per_op != bf_single


@pytest.mark.parametrize("case", R9_CASES)
def test_rotation_rounds_every_operation(case):
    out, bx0, bx1, per_op, _, _, bf_per_op, _ = case
    split, p, pos = (24, 20, 20), 27, np.array([[0, 0, 100]], dtype=np.int32)
    x = np.zeros((1, 1, 64), dtype=np.float32)
    x[0, 0, 2 * p], x[0, 0, 2 * p + 1] = _f32(bx0), _f32(bx1)
    y = rotate_f32(x, pos, split, 10000.0)[0, 0, 2 * p + out]
    assert _bits(y) == per_op
    yb = apply_rope(x, pos, split, 10000.0, "bf16")[0, 0, 2 * p + out]
    assert int(np.asarray(yb).view(np.uint16)) == bf_per_op
