"""3D rotary position embedding (oracle; test infrastructure).

[WF] §4.2 applies RoPE to K before publishing it; the pages name no formula,
so the plainest reading is the textbook rotary embedding applied per video
axis: the head dimension is cut into contiguous sub-bands (t, h, w) of widths
(d_t, d_h, d_w), and inside the sub-band of axis a the element pair
(2i, 2i+1) is rotated by the angle

    phi = pos_a * theta ** (-2 i / d_a),      0 <= i < d_a / 2.

Precision (the stated reading that makes CPU and GPU agree bit for bit):
  1. the exponent -2i/d_a, the power, the angle, cos and sin in float64;
  2. cos and sin rounded to float32;
  3. y0 = x0*c - x1*s and y1 = x0*s + x1*c in float32, every product and
     the sum rounded separately (no fused multiply-add);
  4. y rounded to the storage type (bfloat16: nearest, ties to even).
"""
from __future__ import annotations

import numpy as np

from .numerics import from_f32


def axis_of_pair(p: int, split) -> tuple:
    """(axis, i) for pair index p of the head: axis 0/1/2 = t/h/w and i the
    pair index inside that axis's sub-band."""
    d_t, d_h, d_w = split
    if 2 * p < d_t:
        return 0, p
    if 2 * p < d_t + d_h:
        return 1, p - d_t // 2
    return 2, p - (d_t + d_h) // 2


def pair_factors(pos: np.ndarray, split, theta: float):
    """float32 (cos, sin) of shape [n_tok, D/2] for int positions [n_tok, 3]."""
    d = sum(split)
    pos = np.asarray(pos, dtype=np.int64)
    n = pos.shape[0]
    cos = np.empty((n, d // 2), dtype=np.float32)
    sin = np.empty((n, d // 2), dtype=np.float32)
    for p in range(d // 2):
        a, i = axis_of_pair(p, split)
        exponent = (-2.0 * i) / float(split[a])
        omega = np.power(np.float64(theta), np.float64(exponent))
        phi = pos[:, a].astype(np.float64) * omega
        cos[:, p] = np.cos(phi).astype(np.float32)
        sin[:, p] = np.sin(phi).astype(np.float32)
    return cos, sin


def rotate_f32(x: np.ndarray, pos: np.ndarray, split, theta: float) -> np.ndarray:
    """Rotate float32 x [n_tok, H, D] by positions [n_tok, 3]; float32 result
    (steps 1-3 above)."""
    x = np.asarray(x, dtype=np.float32)
    cos, sin = pair_factors(pos, split, theta)
    c = cos[:, None, :]
    s = sin[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    # numpy evaluates each float32 product and difference with one rounding:
    # no contraction into fused multiply-adds.
    y0 = np.subtract(np.multiply(x0, c, dtype=np.float32),
                     np.multiply(x1, s, dtype=np.float32), dtype=np.float32)
    y1 = np.add(np.multiply(x0, s, dtype=np.float32),
                np.multiply(x1, c, dtype=np.float32), dtype=np.float32)
    y = np.empty_like(x)
    y[..., 0::2] = y0
    y[..., 1::2] = y1
    return y


def apply_rope(x_f32: np.ndarray, pos: np.ndarray, split, theta: float,
               dtype: str) -> np.ndarray:
    """RoPE then rounding to the storage type `dtype` (step 4)."""
    return from_f32(rotate_f32(x_f32, pos, split, theta), dtype)


def rotate_f64(x: np.ndarray, pos: np.ndarray, split, theta: float) -> np.ndarray:
    """The same rotation entirely in float64 (for property checks only)."""
    x = np.asarray(x, dtype=np.float64)
    d = sum(split)
    y = np.empty_like(x)
    pos = np.asarray(pos, dtype=np.int64)
    for p in range(d // 2):
        a, i = axis_of_pair(p, split)
        phi = pos[:, a] * float(theta) ** ((-2.0 * i) / split[a])
        c = np.cos(phi)[:, None]
        s = np.sin(phi)[:, None]
        x0 = x[..., 2 * p]
        x1 = x[..., 2 * p + 1]
        y[..., 2 * p] = x0 * c - x1 * s
        y[..., 2 * p + 1] = x0 * s + x1 * c
    return y
