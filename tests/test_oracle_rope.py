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
